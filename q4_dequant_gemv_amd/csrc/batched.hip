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
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kMfmaWaves = 8;          // 512 threads per block
// 16-row weight tiles per wave: two for up to 32 tokens, one above (registers)
template <int MT>
constexpr int mfma_tiles_n() { return MT <= 2 ? 2 : 1; }
template <int MT>
constexpr int mfma_rows() { return kMfmaWaves * mfma_tiles_n<MT>() * 16; }
constexpr int kStageK = 128;           // activations per LDS stage: half a super-block
constexpr int kARowHalves = kStageK + 8;  // staged token row, padded by 16 bytes

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

// f16 bit patterns of 1024 + sc*q for the two codes of a nibble pair (one
// packed 16-bit multiply-add: sc*q <= 945 fits the 10-bit fraction of 1024).
__device__ __forceinline__ uint32_t pair_operand(uint32_t pair, uint32_t sc2) {
    const u16x2_t p = __builtin_bit_cast(u16x2_t, pair);
    const u16x2_t s = __builtin_bit_cast(u16x2_t, sc2);
    const u16x2_t magic = {0x6400, 0x6400};
    return __builtin_bit_cast(uint32_t, static_cast<u16x2_t>(p * s + magic));
}

// ---- activations, converted once per call ----------------------------------
// For every stage s (activations [128 s, 128 s + 128)) the scratch holds one
// block of stage_bytes(m) bytes, laid out exactly as the LDS copy consumes it:
//   hi[m][128]  f16 of x * 2^-e in staged order (stage_pos)
//   lo[m][128]  f16 of the remainder
//   sub[m][4]   f32 sums of (hi + lo) over each of the stage's four sub-blocks
//   bias[m4]    f32 sum of (hi + lo) over the stage           (m4 = m rounded up to 4)
//   escale[m4]  f32 2^e (0: all zero; NaN: a non-finite input)
__host__ __device__ constexpr int64_t stage_bytes(int m) {
    return ((static_cast<int64_t>(m) * 528 + 8 * ((m + 3) / 4 * 4 / 4) * 4 + 15) / 16) * 16;
}

// One half-wave per (stage, token); each lane converts four activations.  The
// same kernel zero-fills y, which the matrix-core kernel then accumulates into.
__global__ __launch_bounds__(256) void x_prep_kernel(const float *x, uint8_t *__restrict__ xc, float *__restrict__ y,
                                                      int m, int64_t k, int64_t ny) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    for (int64_t i = gid; i < ny; i += static_cast<int64_t>(gridDim.x) * 256) y[i] = 0.0f;

    const int64_t nst = k / kStageK;
    const int64_t pairs = nst * m;
    const int c = threadIdx.x & 31;
    int64_t pair = gid >> 5;
    const bool live = pair < pairs;
    if (!live) pair = pairs - 1;  // keep the half-wave's shuffles uniform; no writes
    const int64_t st = pair / m;
    const int tok = static_cast<int>(pair % m);
    const float *px = x + static_cast<int64_t>(tok) * k + st * kStageK + 4 * c;
    float v[4];
    float amax = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        v[b] = px[b];
        float a = fabsf(v[b]);
        a = (a <= FLT_MAX) ? a : INFINITY;
        amax = fmaxf(amax, a);
    }
    amax = lane_group_max<32>(amax);
    const bool finite = amax <= FLT_MAX;
    const bool nz = finite && amax > 0.0f;
    const int e = nz ? ilogbf(amax) : 0;
    _Float16 hi[4], lo[4];
    float part = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float sv = nz ? ldexpf(v[b], -e) : 0.0f;
        hi[b] = static_cast<_Float16>(sv);
        lo[b] = static_cast<_Float16>(sv - static_cast<float>(hi[b]));
        part += static_cast<float>(hi[b]) + static_cast<float>(lo[b]);
    }
    const float sub8 = lane_group_sum<8>(part);
    const float tot = lane_group_sum<32>(part);
    if (!live) return;
    uint8_t *blk = xc + st * stage_bytes(m);
    const int m4 = (m + 3) / 4 * 4;
    const int pos = stage_pos(4 * c);  // activations 4c..4c+3 land at pos + {0, 2, 1, 3}
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<half4_t *>(blk + (static_cast<int64_t>(tok) * 128 + pos) * 2) = half4_t{hi[0], hi[2], hi[1], hi[3]};
    *reinterpret_cast<half4_t *>(blk + (static_cast<int64_t>(m + tok) * 128 + pos) * 2) =
        half4_t{lo[0], lo[2], lo[1], lo[3]};
    float *sub = reinterpret_cast<float *>(blk + static_cast<int64_t>(m) * 512);
    float *bias = sub + 4 * m;
    float *esc = bias + m4;
    if ((c & 7) == 0) sub[4 * tok + (c >> 3)] = sub8;
    if (c == 0) {
        bias[tok] = tot;
        esc[tok] = finite ? (nz ? ldexpf(1.0f, e) : 0.0f) : NAN;
    }
}

template <int NT>
struct StageW {
    uint4 hdr[NT];
    uint4 q[NT];
};

// Per-block LDS: one stage of activations for 16*MT tokens (rows >= m stay 0).
template <int MT>
struct MfmaShared {
    alignas(16) _Float16 a_hi[16 * MT][kARowHalves];
    alignas(16) _Float16 a_lo[16 * MT][kARowHalves];
    alignas(16) float sub[16 * MT][4];
    alignas(16) float bias[16 * MT];
    alignas(16) float escale[16 * MT];
};

// 16-byte chunks of one stage block: hi rows, lo rows, sub, bias, escale.
__device__ __forceinline__ int stage_chunks(int m) { return 33 * m + (m + 3) / 4 * 2; }

// y += W x over a stream-K share of the (row block, super-block) units: block
// b owns units [b U / G, (b+1) U / G) in row-block-major order and adds its
// partial tiles into y (zero-filled by x_prep_kernel) whenever the row block
// changes.
template <int MT>
__global__ __launch_bounds__(512, 2) void batched_mfma_kernel(const uint8_t *__restrict__ w,
                                                              const uint8_t *__restrict__ xc, float *__restrict__ y,
                                                              int m, int64_t n, int64_t k, int64_t row_bytes) {
    constexpr int NT = mfma_tiles_n<MT>();
    constexpr int kRows = mfma_rows<MT>();
    constexpr int kCopyPerThread = (33 * 16 * MT + 8 * MT + 511) / 512;
    __shared__ __align__(16) MfmaShared<MT> sh;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kq = lane >> 4;

    const int nsb = static_cast<int>(k / kBlockWeights);
    const int64_t nrb = (n + kRows - 1) / kRows;
    const int64_t units = nrb * nsb;
    const int64_t u0 = units * blockIdx.x / gridDim.x;
    const int64_t u1 = units * (blockIdx.x + 1) / gridDim.x;

    // tokens >= m are never copied: clear the whole stage area once
    for (int i = threadIdx.x; i < static_cast<int>(sizeof(MfmaShared<MT>) / 4); i += 512)
        reinterpret_cast<float *>(&sh)[i] = 0.0f;

    // ---- stage copy: chunk q of the scratch block -> fixed LDS address
    const int nchunks = stage_chunks(m);
    const int m4 = (m + 3) / 4 * 4;
    uint32_t src_off[kCopyPerThread];
    uint8_t *dst[kCopyPerThread];
    bool cp_ok[kCopyPerThread];
#pragma unroll
    for (int j = 0; j < kCopyPerThread; ++j) {
        const int q = threadIdx.x + 512 * j;
        cp_ok[j] = q < nchunks;
        const int qq = cp_ok[j] ? q : 0;
        src_off[j] = static_cast<uint32_t>(qq) * 16u;
        uint8_t *d;
        if (qq < 16 * m) d = reinterpret_cast<uint8_t *>(&sh.a_hi[qq >> 4][8 * (qq & 15)]);
        else if (qq < 32 * m) d = reinterpret_cast<uint8_t *>(&sh.a_lo[(qq - 16 * m) >> 4][8 * (qq & 15)]);
        else if (qq < 33 * m) d = reinterpret_cast<uint8_t *>(&sh.sub[qq - 32 * m][0]);
        else if (qq < 33 * m + m4 / 4) d = reinterpret_cast<uint8_t *>(&sh.bias[4 * (qq - 33 * m)]);
        else d = reinterpret_cast<uint8_t *>(&sh.escale[4 * (qq - 33 * m - m4 / 4)]);
        dst[j] = d;
    }
    const int64_t sbytes = stage_bytes(m);
    const int64_t xc_bytes = sbytes * (k / kStageK);
    struct StageC {
        uint4 v[kCopyPerThread];
    };
    auto load_c = [&](StageC &cs, int64_t st) {
        const __amdgpu_buffer_rsrc_t r = stream_rsrc(xc + st * sbytes, static_cast<int>(sbytes));
#pragma unroll
        for (int j = 0; j < kCopyPerThread; ++j) cs.v[j] = buffer_load16(r, src_off[j]);
    };
    auto store_c = [&](const StageC &cs) {
#pragma unroll
        for (int j = 0; j < kCopyPerThread; ++j)
            if (cp_ok[j]) *reinterpret_cast<uint4 *>(dst[j]) = cs.v[j];
    };

    // ---- weights of unit (rb, sb), half h
    auto load_w = [&](StageW<NT> &ws, int64_t u, int h) {
        const int64_t rb = u / nsb;
        const int sb = static_cast<int>(u - rb * nsb);
        const int64_t row0 = rb * kRows;
        const int64_t rows_here = min<int64_t>(kRows, n - row0);
        const __amdgpu_buffer_rsrc_t wr = stream_rsrc(w + row0 * row_bytes, static_cast<int>(rows_here * row_bytes));
        const int soff = sb * kBlockBytes;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t vrow = static_cast<uint32_t>((wave * NT * 16 + t * 16 + col) * row_bytes);
            const u32x4_t q = __builtin_amdgcn_raw_buffer_load_b128(wr, static_cast<int>(vrow + 16 + 64 * h + 16 * kq),
                                                                     soff, 0);
            ws.q[t] = make_uint4(q.x, q.y, q.z, q.w);
            if (h == 0) {
                const u32x4_t hd = __builtin_amdgcn_raw_buffer_load_b128(wr, static_cast<int>(vrow), soff, 0);
                ws.hdr[t] = make_uint4(hd.x, hd.y, hd.z, hd.w);
            }
        }
    };

    const PairSelect psel0 = pair_select(kq >> 1);
    const PairSelect psel1 = pair_select(2 + (kq >> 1));

    float4_t acc[NT][MT];
    auto zero_acc = [&]() {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int p = 0; p < MT; ++p) acc[t][p] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    };
    auto flush = [&](int64_t rb) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int64_t row = rb * kRows + wave * NT * 16 + t * 16 + col;
#pragma unroll
            for (int p = 0; p < MT; ++p) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tok = 16 * p + 4 * kq + r;
                    if (row < n && tok < m) unsafeAtomicAdd(&y[static_cast<int64_t>(tok) * n + row], acc[t][p][r]);
                }
            }
        }
    };

    auto compute = [&](const StageW<NT> &ws, const uint4 (&hdr)[NT], int h) {
        const PairSelect &ps = h ? psel1 : psel0;
        const int gg = kq >> 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float dd = half_bits_to_float(hdr[t].x);
            const float dm = half_bits_to_float(hdr[t].x >> 16);
            uint32_t scp, mp;
            scale_min_pair(hdr[t].y, hdr[t].z, hdr[t].w, ps, scp, mp);
            const uint32_t sc2_lo = (scp & 0xffu) * 0x00010001u;
            const uint32_t sc2_hi = ((scp >> 8) & 0xffu) * 0x00010001u;
            const uint32_t u[4] = {ws.q[t].x, ws.q[t].y, ws.q[t].z, ws.q[t].w};
            half8_t bop[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sc2 = (i & 1) ? sc2_hi : sc2_lo;
                const int shn = (i & 1) ? 4 : 0;
                uint32_t v4[4];
#pragma unroll
                for (int d2 = 0; d2 < 2; ++d2) {
                    const uint32_t word = u[2 * (i >> 1) + d2];
                    v4[2 * d2 + 0] = pair_operand((word >> shn) & 0x000f000fu, sc2);
                    v4[2 * d2 + 1] = pair_operand((word >> (8 + shn)) & 0x000f000fu, sc2);
                }
                bop[i] = __builtin_bit_cast(half8_t, u32x4_t{v4[0], v4[1], v4[2], v4[3]});
            }
            // mins of the lane's two sub-blocks (even quarters only) as exact f16
            const _Float16 m0 = (kq & 1) ? _Float16(0) : static_cast<_Float16>(static_cast<float>(mp & 0xffu));
            const _Float16 m1 = (kq & 1) ? _Float16(0) : static_cast<_Float16>(static_cast<float>((mp >> 8) & 0xffu));
            const half8_t bmin = {m0, m1, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int p = 0; p < MT; ++p) {
                const int tok = 16 * p + col;
                float4_t pacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const half8_t ahi = *reinterpret_cast<const half8_t *>(&sh.a_hi[tok][kq * 32 + i * 8]);
                    const half8_t alo = *reinterpret_cast<const half8_t *>(&sh.a_lo[tok][kq * 32 + i * 8]);
                    pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi, bop[i], pacc, 0, 0, 0);
                    pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo, bop[i], pacc, 0, 0, 0);
                }
                // sub-block sums of this quarter's group as the A operand of the min product
                const float s0 = sh.sub[tok][2 * gg], s1 = sh.sub[tok][2 * gg + 1];
                const _Float16 s0h = static_cast<_Float16>(s0), s1h = static_cast<_Float16>(s1);
                const _Float16 s0l = static_cast<_Float16>(s0 - static_cast<float>(s0h));
                const _Float16 s1l = static_cast<_Float16>(s1 - static_cast<float>(s1h));
                const half8_t shi = {s0h, s1h, 0, 0, 0, 0, 0, 0};
                const half8_t slo = {s0l, s1l, 0, 0, 0, 0, 0, 0};
                float4_t qacc = {0.0f, 0.0f, 0.0f, 0.0f};
                qacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(shi, bmin, qacc, 0, 0, 0);
                qacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(slo, bmin, qacc, 0, 0, 0);
                // pacc[r] = sum_k A[tok_r, k] * (1024 + sc q)[k, col]; tok_r = 16p + 4kq + r
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = 16 * p + 4 * kq + r;
                    const float code_part = pacc[r] - 1024.0f * sh.bias[tr];
                    acc[t][p][r] += sh.escale[tr] * (dd * code_part - dm * qacc[r]);
                }
                // one token tile's operands live at a time (register budget)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    zero_acc();
    if (u0 >= u1) return;
    // Pipeline: the weights and activations of the next half block are loaded
    // while the current one is multiplied.  Loads past the last unit re-read
    // the last unit (unused).
    StageC ca, cb;
    StageW<NT> wa, wb;
    int64_t cur_rb = u0 / nsb;
    load_c(ca, 2 * (u0 % nsb));
    load_w(wa, u0, 0);
    for (int64_t u = u0; u < u1; ++u) {
        const int64_t rb = u / nsb;
        const int sb = static_cast<int>(u - rb * nsb);
        if (rb != cur_rb) {
            flush(cur_rb);
            zero_acc();
            cur_rb = rb;
        }
        // half 0
        load_c(cb, 2 * sb + 1);
        load_w(wb, u, 1);
        __syncthreads();
        store_c(ca);
        __syncthreads();
        compute(wa, wa.hdr, 0);
        // half 1 (headers of this super-block still in wa)
        uint4 hdr[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) hdr[t] = wa.hdr[t];
        const int64_t un = u + 1 < u1 ? u + 1 : u;
        load_c(ca, 2 * (un % nsb));
        load_w(wa, un, 0);
        __syncthreads();
        store_c(cb);
        __syncthreads();
        compute(wb, hdr, 1);
    }
    flush(cur_rb);
    (void)xc_bytes;
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
hipError_t launch_mfma(const uint8_t *w, const float *x, float *y, int m, int64_t n, int64_t k,
                       hipStream_t stream) {
    const int64_t nst = k / kStageK;
    const int64_t bytes = stage_bytes(m) * nst;
    uint8_t *xc = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void **>(&xc), static_cast<size_t>(bytes), stream);
    if (e != hipSuccess) return e;
    const int64_t prep_threads = nst * m * 32;
    const int64_t prep_blocks = (prep_threads + 255) / 256;
    hipLaunchKernelGGL(x_prep_kernel, dim3(static_cast<unsigned>(prep_blocks)), dim3(256), 0, stream, x, xc, y, m, k,
                       static_cast<int64_t>(m) * n);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int grid = device_cu_count();
        hipLaunchKernelGGL(batched_mfma_kernel<MT>, dim3(grid), dim3(512), 0, stream, w, xc, y, m, n, k,
                           (k / kBlockWeights) * kBlockBytes);
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(xc, stream);
    return e != hipSuccess ? e : f;
}

}  // namespace

hipError_t launch_gemv_batched(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                               hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (k == 0) return launch_fill_zero(y, m * n, stream);
    if (m == 1) return launch_gemv(w, nullptr, x, y, n, k, stream);
    if (m < 16) return dispatch_valu(w, x, y, m, n, k, stream);
    hipError_t e = hipSuccess;
    // up to 64 tokens per launch; the weights are re-read per 64-token slice
    for (int64_t t0 = 0; t0 < m; t0 += 64) {
        const int mt = static_cast<int>(m - t0 < 64 ? m - t0 : 64);
        const float *xs = x + t0 * k;
        float *ys = y + t0 * n;
        if (mt <= 16) e = launch_mfma<1>(w, xs, ys, mt, n, k, stream);
        else if (mt <= 32) e = launch_mfma<2>(w, xs, ys, mt, n, k, stream);
        else if (mt <= 48) e = launch_mfma<3>(w, xs, ys, mt, n, k, stream);
        else e = launch_mfma<4>(w, xs, ys, mt, n, k, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace q4k
