// Skinny Q4_K GEMM: y[t, r] = sum_c W[r,c] x[t,c] for m tokens.
//
// selectQ4KFusedVariant ("@simulatte/doppler 0.1.7 -> 0.1.8",
// matmul-selection.js) picks a fused Q4K kernel by whether M == 1; this file
// is the M > 1 side.  Two kernels:
//
//  * m < 16, vector ALUs.  A workgroup owns 64 rows and walks K in chunks of
//    1024 activations; per chunk the m activation rows are converted to the
//    integer limbs of q4k_int_dot.h and staged in LDS, and each 64-weight group
//    of codes is decoded once and multiplied against all m activation rows
//    (v_dot4_i32_i8), so a weight byte is read from HBM once per call.
//
//  * m >= 16, matrix cores.  Only here is the work a real dense contraction,
//    so the codes are turned into f16 MFMA operands: the B operand holds
//    1024 + sc*q (exact in f16 since sc*q <= 945 < 1024, built with one packed
//    16-bit multiply-add per two codes), which folds each sub-block's six-bit
//    scale into the operand so that a whole half super-block (4 sub-blocks,
//    128 weights) accumulates into one f32 tile.  Activations enter as f16
//    hi + lo parts of x * 2^-e (e per token and half super-block), so the
//    products are exact and the tile carries f32 accuracy.  Per half super-
//    block the tile is finished in f32: subtract the 1024 * sum(x) bias, scale
//    by d and 2^e, subtract dmin * sum_s m_s * sum(x over s).
//    v_mfma_f32_16x16x32_f16: 16 tokens x 16 rows x 32 weights per step.
//    (A bf16 operand cannot hold sc*q exactly -- 8 significant bits -- and a
//    bf16 dequantized weight misses the 2e-4 * sum|w x| bound at K = 4096.)
#include <float.h>
#include <math.h>

#include "launch.h"
#include "q4k_device.h"
#include "q4k_int_dot.h"

namespace q4k {

// ------------------------------------------------------------ m < 16 (VALU)
constexpr int kValuChunkGroups = 16;  // 1024 activations per LDS chunk
constexpr int kValuRowsPerBlock = 64;

template <int M>
__global__ __launch_bounds__(256) void batched_valu_kernel(const uint8_t *__restrict__ w,
                                                           const float *__restrict__ x, float *__restrict__ y,
                                                           int64_t n, int64_t k, int64_t row_bytes) {
    __shared__ XGroup xg[M][kValuChunkGroups];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & 15;   // group inside the chunk
    const int slot = lane >> 4;  // row inside a pass of four rows
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kValuRowsPerBlock + wave * 16;
    const int ngroups = static_cast<int>(k / 64);

    float acc[4][M];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int t = 0; t < M; ++t) acc[p][t] = 0.0f;

    for (int g0 = 0; g0 < ngroups; g0 += kValuChunkGroups) {
        const int cg = min(kValuChunkGroups, ngroups - g0);
        __syncthreads();
        for (int t = 0; t < M; ++t) prepare_x<256>(x + t * k + 64 * g0, cg, &xg[t][0]);
        __syncthreads();
        const int j = g0 + sub;
        const bool gok = sub < cg;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t row = row0 + 4 * p + slot;
            if (row < n && gok) {
                const uint8_t *blk = w + row * row_bytes + (j >> 2) * kBlockBytes;
                const int grp = j & 3;
                const uint4 hdr = load_stream16(blk);
                const uint4 qa = load_stream16(blk + 16 + 32 * grp);
                const uint4 qb = load_stream16(blk + 32 + 32 * grp);
                GroupCodes c;
                decode_group(hdr, qa, qb, pair_select(grp), c);
#pragma unroll
                for (int t = 0; t < M; ++t) acc[p][t] += xg[t][sub].scale * group_dot(c, xg[t][sub]);
            }
        }
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t row = row0 + 4 * p + slot;
#pragma unroll
        for (int t = 0; t < M; ++t) {
            const float v = group_sum<16>(acc[p][t]);
            if (sub == 0 && row < n) y[t * n + row] = v;
        }
    }
}

// ------------------------------------------------------- m >= 16 (MFMA)
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

constexpr int kStageK = 128;                // half super-block per LDS stage
constexpr int kARowHalves = kStageK + 8;    // f16 per staged token row (16 B pad)

// Position of in-stage activation kk (0..127) inside a staged token row: the
// order in which the B operand below consumes the codes.  A lane-quarter kq
// (lanes 16kq..16kq+15) owns code bytes [16kq, 16kq+16) of the half block's 64
// code bytes: group 2h + kq/2, bytes 16*(kq%2).. of that group.  Its dword d
// (bytes 4d..4d+3) splits into the nibble pairs (byte0, byte2) and
// (byte1, byte3); MFMA step i takes the low (i even) or high (i odd) nibbles
// of dwords 2*(i/2) and 2*(i/2)+1.
__device__ __forceinline__ int stage_pos(int kk) {
    const int gg = kk >> 6;
    const int r = kk & 63;
    const int sd = r >> 5;     // 0: low nibble (sub-block 2g), 1: high nibble
    const int l = r & 31;      // code byte inside the group
    const int kq = 2 * gg + (l >> 4);
    const int lo = l & 15;
    const int dd = lo >> 2;
    const int b = lo & 3;
    const int i = 2 * (dd >> 1) + sd;
    const int tb = (b == 1) ? 2 : (b == 2) ? 1 : b;
    return kq * 32 + i * 8 + 4 * (dd & 1) + tb;
}

// f16 bit patterns of 1024 + sc*q for the two codes of a nibble pair.
__device__ __forceinline__ uint32_t pair_operand(uint32_t pair, uint32_t sc2) {
    const u16x2_t p = __builtin_bit_cast(u16x2_t, pair);
    const u16x2_t s = __builtin_bit_cast(u16x2_t, sc2);
    const u16x2_t magic = {0x6400, 0x6400};
    return __builtin_bit_cast(uint32_t, static_cast<u16x2_t>(p * s + magic));
}

template <int MT>
__global__ __launch_bounds__(256) void batched_mfma_kernel(const uint8_t *__restrict__ w,
                                                           const float *__restrict__ x, float *__restrict__ y,
                                                           int m, int64_t n, int64_t k, int64_t row_bytes,
                                                           int64_t ldy) {
    constexpr int kTokens = 16 * MT;
    __shared__ __align__(16) _Float16 a_hi[kTokens][kARowHalves];
    __shared__ __align__(16) _Float16 a_lo[kTokens][kARowHalves];
    __shared__ float s_bias[kTokens];     // sum over the stage of (hi + lo)
    __shared__ float s_sub[kTokens][4];   // per sub-block sums of (hi + lo)
    __shared__ float s_exp[kTokens];      // 2^e of the stage (0: all zero, NaN: non-finite)

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;  // row of W inside the wave's 16-row tile
    const int kq = lane >> 4;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 64 + wave * 16 + col;
    const bool rok = row < n;
    const uint8_t *wrow = w + (rok ? row : 0) * row_bytes;

    float4_t acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int64_t nsb = k / kBlockWeights;
    for (int64_t sb = 0; sb < nsb; ++sb) {
        uint4 hdr = make_uint4(0, 0, 0, 0);
        if (rok) hdr = load_stream16(wrow + sb * kBlockBytes);
        const float d = half_bits_to_float(hdr.x);
        const float dmin = half_bits_to_float(hdr.x >> 16);
#pragma unroll 1
        for (int h = 0; h < 2; ++h) {
            // ---- stage activations [sb*256 + 128h, +128) of every token
            __syncthreads();
            for (int tok = threadIdx.x >> 5; tok < kTokens; tok += 8) {
                const int c = threadIdx.x & 31;
                const int kk = 4 * c;
                float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                if (tok < m) {
                    const float *p = x + static_cast<int64_t>(tok) * k + sb * kBlockWeights + kStageK * h + kk;
#pragma unroll
                    for (int b = 0; b < 4; ++b) v[b] = p[b];
                }
                float amax = 0.0f;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    float a = fabsf(v[b]);
                    a = (a <= FLT_MAX) ? a : INFINITY;
                    amax = fmaxf(amax, a);
                }
                amax = group_max<32>(amax);
                const bool finite = amax <= FLT_MAX;
                int e = 0;
                float sexp = 0.0f;
                if (!finite) {
                    sexp = NAN;
                } else if (amax > 0.0f) {
                    e = ilogbf(amax);
                    sexp = ldexpf(1.0f, e);
                }
                _Float16 hi[4], lo[4];
                float part = 0.0f;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float s = (finite && amax > 0.0f) ? ldexpf(v[b], -e) : 0.0f;
                    hi[b] = static_cast<_Float16>(s);
                    lo[b] = static_cast<_Float16>(s - static_cast<float>(hi[b]));
                    part += static_cast<float>(hi[b]) + static_cast<float>(lo[b]);
                }
                const int pos = stage_pos(kk);  // kk..kk+3 land at pos + {0, 2, 1, 3}
                a_hi[tok][pos + 0] = hi[0];
                a_hi[tok][pos + 2] = hi[1];
                a_hi[tok][pos + 1] = hi[2];
                a_hi[tok][pos + 3] = hi[3];
                a_lo[tok][pos + 0] = lo[0];
                a_lo[tok][pos + 2] = lo[1];
                a_lo[tok][pos + 1] = lo[2];
                a_lo[tok][pos + 3] = lo[3];
                const float sub8 = group_sum<8>(part);  // the 32 activations of one sub-block
                if ((c & 7) == 0) s_sub[tok][c >> 3] = sub8;
                const float tot = group_sum<32>(part);
                if (c == 0) {
                    s_bias[tok] = tot;
                    s_exp[tok] = sexp;
                }
            }
            __syncthreads();

            // ---- B operand: this lane's 16 code bytes of the half block
            uint4 q = make_uint4(0, 0, 0, 0);
            if (rok) q = load_stream16(wrow + sb * kBlockBytes + 16 + 64 * h + 16 * kq);
            const int g = 2 * h + (kq >> 1);
            int sc_lo, m_lo, sc_hi, m_hi;
            scale_min(hdr.y, hdr.z, hdr.w, 2 * g, sc_lo, m_lo);
            scale_min(hdr.y, hdr.z, hdr.w, 2 * g + 1, sc_hi, m_hi);
            const uint32_t sc2_lo = static_cast<uint32_t>(sc_lo) * 0x00010001u;
            const uint32_t sc2_hi = static_cast<uint32_t>(sc_hi) * 0x00010001u;
            const uint32_t u[4] = {q.x, q.y, q.z, q.w};
            half8_t bop[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sc2 = (i & 1) ? sc2_hi : sc2_lo;
                const int sh = (i & 1) ? 4 : 0;
                uint32_t v4[4];
#pragma unroll
                for (int dd = 0; dd < 2; ++dd) {
                    const uint32_t word = u[2 * (i >> 1) + dd];
                    v4[2 * dd + 0] = pair_operand((word >> sh) & 0x000f000fu, sc2);
                    v4[2 * dd + 1] = pair_operand((word >> (8 + sh)) & 0x000f000fu, sc2);
                }
                typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
                bop[i] = __builtin_bit_cast(half8_t, u32x4_t{v4[0], v4[1], v4[2], v4[3]});
            }
            // the four mins of this half block's sub-blocks, for this lane's row
            float mins[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                int scs, ms;
                scale_min(hdr.y, hdr.z, hdr.w, 4 * h + s, scs, ms);
                mins[s] = static_cast<float>(ms);
            }

#pragma unroll
            for (int t = 0; t < MT; ++t) {
                float4_t p = {0.0f, 0.0f, 0.0f, 0.0f};
                const int tok = 16 * t + (lane & 15);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const half8_t ah = *reinterpret_cast<const half8_t *>(&a_hi[tok][kq * 32 + i * 8]);
                    const half8_t al = *reinterpret_cast<const half8_t *>(&a_lo[tok][kq * 32 + i * 8]);
                    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bop[i], p, 0, 0, 0);
                    p = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bop[i], p, 0, 0, 0);
                }
                // p[r] = sum_k A[tok_r, k] * (1024 + sc q)[k, col], tok_r = 16t + 4*kq + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 16 * t + 4 * kq + r;
                    const float code_part = p[r] - 1024.0f * s_bias[tr];
                    const float min_part = mins[0] * s_sub[tr][0] + mins[1] * s_sub[tr][1] +
                                           mins[2] * s_sub[tr][2] + mins[3] * s_sub[tr][3];
                    acc[t][r] += s_exp[tr] * (d * code_part - dmin * min_part);
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = 16 * t + 4 * kq + r;
            if (rok && tok < m) y[static_cast<int64_t>(tok) * ldy + row] = acc[t][r];
        }
    }
}

// ------------------------------------------------------------- launchers
namespace {

template <int M>
hipError_t launch_valu(const uint8_t *w, const float *x, float *y, int64_t n, int64_t k, hipStream_t stream) {
    const int64_t grid = (n + kValuRowsPerBlock - 1) / kValuRowsPerBlock;
    hipLaunchKernelGGL(batched_valu_kernel<M>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, w, x, y, n, k,
                       (k / kBlockWeights) * kBlockBytes);
    return hipGetLastError();
}

hipError_t dispatch_valu(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                         hipStream_t stream) {
    switch (m) {
        case 2: return launch_valu<2>(w, x, y, n, k, stream);
        case 3: return launch_valu<3>(w, x, y, n, k, stream);
        case 4: return launch_valu<4>(w, x, y, n, k, stream);
        case 5: return launch_valu<5>(w, x, y, n, k, stream);
        case 6: return launch_valu<6>(w, x, y, n, k, stream);
        case 7: return launch_valu<7>(w, x, y, n, k, stream);
        case 8: return launch_valu<8>(w, x, y, n, k, stream);
        case 9: return launch_valu<9>(w, x, y, n, k, stream);
        case 10: return launch_valu<10>(w, x, y, n, k, stream);
        case 11: return launch_valu<11>(w, x, y, n, k, stream);
        case 12: return launch_valu<12>(w, x, y, n, k, stream);
        case 13: return launch_valu<13>(w, x, y, n, k, stream);
        case 14: return launch_valu<14>(w, x, y, n, k, stream);
        default: return launch_valu<15>(w, x, y, n, k, stream);
    }
}

template <int MT>
hipError_t launch_mfma(const uint8_t *w, const float *x, float *y, int m, int64_t n, int64_t k, int64_t ldy,
                       hipStream_t stream) {
    const int64_t grid = (n + 63) / 64;
    hipLaunchKernelGGL(batched_mfma_kernel<MT>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, w, x, y, m,
                       n, k, (k / kBlockWeights) * kBlockBytes, ldy);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_batched(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                               hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (k == 0) return launch_fill_zero(y, m * n, stream);
    if (m == 1) return launch_gemv(w, nullptr, x, y, n, k, stream);
    if (m < 16) return dispatch_valu(w, x, y, m, n, k, stream);
    // up to 64 tokens per launch; the weights are re-read per 64-token slice
    for (int64_t t0 = 0; t0 < m; t0 += 64) {
        const int mt = static_cast<int>(m - t0 < 64 ? m - t0 : 64);
        const float *xs = x + t0 * k;
        float *ys = y + t0 * n;
        hipError_t e;
        if (mt <= 16) e = launch_mfma<1>(w, xs, ys, mt, n, k, n, stream);
        else if (mt <= 32) e = launch_mfma<2>(w, xs, ys, mt, n, k, n, stream);
        else if (mt <= 48) e = launch_mfma<3>(w, xs, ys, mt, n, k, n, stream);
        else e = launch_mfma<4>(w, xs, ys, mt, n, k, n, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4k
