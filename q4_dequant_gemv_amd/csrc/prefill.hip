// Prefill-size Q4_K GEMM with f16 activations (W4A16):
//     y[t, r] = sum_c W[r,c] x[t,c],   x f16 [m, k], y f32 or f16 [m, n].
//
// The prefill side of the phase choice in "@simulatte/doppler 0.1.7 ->
// 0.1.8" (matmul-selection.js: resolveMatmulPhase treats M > 1 as prefill,
// selectQ4KFusedVariant takes the activation dtype); "Module qwen3_attention"
// names the W4A16 batched dispatcher this corresponds to.  With hundreds of
// tokens sharing every weight the work is a dense contraction bound by the
// matrix cores, so the design goal is to keep them fed.
//
// Operands (exact, so the f32 accumulation is the only rounding):
//   * A = the f16 activations themselves.
//   * B = sc * q of sub-block j (at most 63 * 15 = 945, an integer, exact in
//     f16), built per MFMA step with one packed 16-bit multiply-add per two
//     codes (1024 + sc*q as an f16 bit pattern) and one packed f16 subtract.
//   * Per super-block s the f32 tile P_s = sum_k x * sc*q (8 MFMA steps of 32
//     weights) is finished as
//         acc += d_s * P_s - dmin_s * Q_s,   Q_s = sum_j m_j * (sum of x over j),
//     where Q_s is one 16x16x16 MFMA: A holds the eight sub-block sums of each
//     token (divided by 32 so they stay inside the f16 range) as hi + lo f16
//     parts, B the eight six-bit mins (exact).
//
// Data flow.  A preparation kernel writes the activations once per call into
// scratch in the lane order of the MFMA operand (and the sub-block sums).  A
// workgroup of 4 waves owns a 128-row x 128-token tile; each wave a 64 x 64
// quarter (4 x 4 tiles of 16 x 16).  K is walked in half super-blocks: the
// workgroup copies the next half super-block of activations (32 KB) and, every
// other step, the next super-block of its 128 weight rows (18 KB) into LDS
// with direct-to-LDS buffer loads while the matrix cores work on the current
// one (double-buffered, one barrier per step).  Every output is computed by
// one lane in a fixed order: results are bitwise reproducible.
#include <type_traits>

#include "launch.h"
#include "q4k_device.h"

namespace q4k {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kPfTile = 128;                  // rows and tokens per workgroup tile
constexpr int kPfHalf = 128;                  // activations per pipeline step (half a super-block)
constexpr int kAStage = 8 * 4 * 64 * 16;      // [token tile][MFMA step][lane][8 f16] = 32 KB
constexpr int kWStage = kPfTile * kBlockBytes;  // one super-block of 128 rows = 18 KB
constexpr int kMinBlock = 8 * 64 * 8;         // [token tile][lane][4 f16] = 4 KB per super-block
constexpr int kWPieces = kWStage / 16;        // 1152 16-byte pieces = 18 wave-wide copies

__device__ __forceinline__ half8_t as_half8(u32x4_t v) { return __builtin_bit_cast(half8_t, v); }

}  // namespace

// ---- activations, once per call ----------------------------------------------
// One thread per 8 consecutive activations of one token (tokens past m are
// zeros).  Writes them, permuted to the order in which the B operand below
// consumes codes (positions 0, 2, 1, 3, 4, 6, 5, 7), at their place in the
// operand fragments; the four threads of a sub-block add up its 32
// activations, and the first of them stores the sum / 32 as hi and lo f16 in
// the min-term operand.
__global__ __launch_bounds__(256) void prefill_prep_kernel(const _Float16 *__restrict__ x, uint8_t *__restrict__ xa,
                                                           uint8_t *__restrict__ xs, int64_t m, int64_t mpad,
                                                           int64_t k) {
    const int64_t chunks = k / 8;
    const int64_t total = mpad * chunks;
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (gid >= total) return;  // whole groups of four: total is a multiple of 4
    const int64_t nblocks = mpad / kPfTile;
    const int64_t t = gid / chunks;
    const int64_t k0 = 8 * (gid % chunks);
    half8_t v = {0, 0, 0, 0, 0, 0, 0, 0};
    if (t < m) v = *reinterpret_cast<const half8_t *>(x + t * k + k0);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) part += static_cast<float>(v[i]);
    const float sub_sum = lane_group_sum<4>(part);  // the sub-block's 32 activations

    const int64_t hsb = k0 / kPfHalf;
    const int sp = static_cast<int>((k0 % kPfHalf) / 32);
    const int kb = static_cast<int>((k0 % 32) / 8);
    const int64_t blk = t / kPfTile;
    const int tile = static_cast<int>((t % kPfTile) / 16);
    const int tl = static_cast<int>(t % 16);
    const half8_t pv = {v[0], v[2], v[1], v[3], v[4], v[6], v[5], v[7]};
    *reinterpret_cast<half8_t *>(xa + (hsb * nblocks + blk) * kAStage + ((tile * 4 + sp) * 64 + tl + 16 * kb) * 16) =
        pv;
    if (kb == 0) {
        const int64_t sb = k0 / kBlockWeights;
        const int sub = static_cast<int>((k0 % kBlockWeights) / 32);
        const float s32 = sub_sum * 0.03125f;
        const _Float16 hi = static_cast<_Float16>(s32);
        const _Float16 lo = static_cast<_Float16>(s32 - static_cast<float>(hi));
        _Float16 *q = reinterpret_cast<_Float16 *>(xs + (sb * nblocks + blk) * kMinBlock);
        q[(tile * 64 + tl + 16 * (sub >> 2)) * 4 + (sub & 3)] = hi;
        q[(tile * 64 + tl + 16 * (2 + (sub >> 2))) * 4 + (sub & 3)] = lo;
    }
}

// ---- the matrix-core kernel ---------------------------------------------------
template <typename YT>
__global__ __launch_bounds__(256, 1) void prefill_mfma_kernel(const uint8_t *__restrict__ w,
                                                              const uint8_t *__restrict__ xa,
                                                              const uint8_t *__restrict__ xs, YT *__restrict__ y,
                                                              int64_t m, int64_t n, int64_t k, int64_t row_bytes,
                                                              int nblocks, int nrb) {
    __shared__ __align__(16) uint8_t a_lds[2][kAStage];
    __shared__ __align__(16) uint8_t w_lds[2][kWStage];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int wr = wave & 1;   // the wave's 64 rows of the tile
    const int wt = wave >> 1;  // the wave's 64 tokens of the tile
    const int col = lane & 15;
    const int kb = lane >> 4;

    const int rbk = static_cast<int>(blockIdx.x % nrb);
    const int tbk = static_cast<int>(blockIdx.x / nrb);
    const int64_t row0 = static_cast<int64_t>(rbk) * kPfTile;
    const int64_t tok0 = static_cast<int64_t>(tbk) * kPfTile;
    const int nsb = static_cast<int>(k / kBlockWeights);
    const int64_t rows_here = n - row0 < kPfTile ? n - row0 : kPfTile;
    // rows past n read as zeros; their results are not stored
    const __amdgpu_buffer_rsrc_t wrs = stream_rsrc(w + row0 * row_bytes, static_cast<int>(rows_here * row_bytes));

    // direct-to-LDS copies: each instruction moves 64 x 16 bytes to LDS
    // base + 16 * lane
    auto dma_a = [&](int h, int buf) {
        const __amdgpu_buffer_rsrc_t ar =
            stream_rsrc(xa + (static_cast<int64_t>(h) * nblocks + tbk) * kAStage, kAStage);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = wave * 8 + i;
            lds_u8 *dst = (lds_u8 *)(&a_lds[buf][0]) + c * 1024;  // generic -> LDS address space
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, reinterpret_cast<lds_void *>(dst), 16, c * 1024 + lane * 16,
                                                     0, 0, 0);
        }
    };
    auto dma_w = [&](int s, int buf) {
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int ii = wave + 4 * i;  // 18 copies over 4 waves
            if (ii < kWPieces / 64) {
                const int p = ii * 64 + lane;
                const int row = p / 9;
                const int pc = p % 9;
                const uint32_t off = static_cast<uint32_t>(row * row_bytes) + static_cast<uint32_t>(s) * kBlockBytes +
                                     static_cast<uint32_t>(pc * 16);
                lds_u8 *dst = (lds_u8 *)(&w_lds[buf][0]) + ii * 1024;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, reinterpret_cast<lds_void *>(dst), 16, off, 0, 0, 0);
            }
        }
    };

    float4_t acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[rt][tt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const half8_t k1024 = {1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024};

    dma_a(0, 0);
    dma_w(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int s = 0; s < nsb; ++s) {
        const uint8_t *wl = w_lds[s & 1];
        // headers of the wave's rows: d, dmin, and the mins as the B operand
        // of the min-term product (k-group kb: sub-blocks 4*(kb&1) .. +3)
        uint4 hdr[4];
        float dd[4], dm[4];
        half4_t qb[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            hdr[rt] = *reinterpret_cast<const uint4 *>(wl + (wr * 64 + rt * 16 + col) * kBlockBytes);
            dd[rt] = half_bits_to_float(hdr[rt].x);
            dm[rt] = 32.0f * half_bits_to_float(hdr[rt].x >> 16);  // the sums are stored / 32
            half4_t mv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                int sc, mm;
                scale_min(hdr[rt].y, hdr[rt].z, hdr[rt].w, 4 * (kb & 1) + q, sc, mm);
                mv[q] = static_cast<_Float16>(static_cast<float>(mm));
            }
            qb[rt] = mv;
        }
        // the wave's tokens' sub-block sums (A of the min-term product)
        half4_t qa[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            qa[tt] = *reinterpret_cast<const half4_t *>(
                xs + (static_cast<int64_t>(s) * nblocks + tbk) * kMinBlock + ((wt * 4 + tt) * 64 + lane) * 8);
        }

        float4_t P[4][4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int h = 2 * s + half;
            if (h + 1 < 2 * nsb) {
                dma_a(h + 1, (h + 1) & 1);
                if (half == 1) dma_w(s + 1, (s + 1) & 1);
            }
            const uint8_t *al = a_lds[half];
            uint2 codes[4];
#pragma unroll
            for (int sp = 0; sp < 4; ++sp) {
                const int j = 4 * half + sp;  // sub-block of the super-block
                half8_t a[4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    a[tt] = *reinterpret_cast<const half8_t *>(al + (((wt * 4 + tt) * 4 + sp) * 64 + lane) * 16);
                if ((sp & 1) == 0) {
                    // 8 code bytes of group j/2 for this lane's k-group
#pragma unroll
                    for (int rt = 0; rt < 4; ++rt)
                        codes[rt] = *reinterpret_cast<const uint2 *>(wl + (wr * 64 + rt * 16 + col) * kBlockBytes + 16 +
                                                                     32 * (j >> 1) + 8 * kb);
                }
                const int shn = (sp & 1) ? 4 : 0;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    int sc, mm;
                    scale_min(hdr[rt].y, hdr[rt].z, hdr[rt].w, j, sc, mm);
                    const uint32_t sc2 = static_cast<uint32_t>(sc) * 0x00010001u;
                    const uint32_t v0 = pair_operand((codes[rt].x >> shn) & 0x000f000fu, sc2);
                    const uint32_t v1 = pair_operand((codes[rt].x >> (8 + shn)) & 0x000f000fu, sc2);
                    const uint32_t v2 = pair_operand((codes[rt].y >> shn) & 0x000f000fu, sc2);
                    const uint32_t v3 = pair_operand((codes[rt].y >> (8 + shn)) & 0x000f000fu, sc2);
                    const half8_t b = as_half8(u32x4_t{v0, v1, v2, v3}) - k1024;  // sc*q, exact
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        P[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], b, j == 0 ? zero : P[rt][tt], 0, 0, 0);
                }
            }
            // the next step's copies have landed; every wave is done with this step's buffers
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        // finish super-block s: acc += d * P - dmin * Q
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float4_t q = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[tt], qb[rt], zero, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rt][tt][r] += dd[rt] * P[rt][tt][r] - dm[rt] * q[r];
            }
        }
    }

    // lane: row col of each row tile, tokens 4*kb .. 4*kb+3 of each token tile
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int64_t row = row0 + wr * 64 + rt * 16 + col;
        if (row >= n) continue;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tok = tok0 + wt * 64 + tt * 16 + kb * 4 + r;
                if (tok < m) y[tok * n + row] = static_cast<YT>(acc[rt][tt][r]);
            }
        }
    }
}

hipError_t launch_prefill(const uint8_t *w, const _Float16 *x, void *y, bool y_f16, int64_t m, int64_t n, int64_t k,
                          hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (k == 0) {
        return y_f16 ? launch_fill_zero_f16(static_cast<_Float16 *>(y), m * n, stream)
                     : launch_fill_zero(static_cast<float *>(y), m * n, stream);
    }
    const int64_t mpad = (m + kPfTile - 1) / kPfTile * kPfTile;
    const int64_t nblocks = mpad / kPfTile;
    const int64_t nrb = (n + kPfTile - 1) / kPfTile;
    const int64_t nsb = k / kBlockWeights;
    const int64_t xa_bytes = mpad * k * 2;
    const int64_t xs_bytes = nsb * nblocks * kMinBlock;
    uint8_t *scratch = nullptr;
    hipError_t e = hipMallocAsync(reinterpret_cast<void **>(&scratch), static_cast<size_t>(xa_bytes + xs_bytes),
                                  stream);
    if (e != hipSuccess) return e;
    uint8_t *xa = scratch;
    uint8_t *xs = scratch + xa_bytes;
    const int64_t prep_threads = mpad * (k / 8);
    hipLaunchKernelGGL(prefill_prep_kernel, dim3(static_cast<unsigned>((prep_threads + 255) / 256)), dim3(256), 0,
                       stream, x, xa, xs, m, mpad, k);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const dim3 grid(static_cast<unsigned>(nrb * nblocks));
        const int64_t rb = (k / kBlockWeights) * kBlockBytes;
        if (y_f16) {
            hipLaunchKernelGGL(prefill_mfma_kernel<_Float16>, grid, dim3(256), 0, stream, w, xa, xs,
                               static_cast<_Float16 *>(y), m, n, k, rb, static_cast<int>(nblocks),
                               static_cast<int>(nrb));
        } else {
            hipLaunchKernelGGL(prefill_mfma_kernel<float>, grid, dim3(256), 0, stream, w, xa, xs,
                               static_cast<float *>(y), m, n, k, rb, static_cast<int>(nblocks), static_cast<int>(nrb));
        }
        e = hipGetLastError();
    }
    const hipError_t f = hipFreeAsync(scratch, stream);
    return e != hipSuccess ? e : f;
}

}  // namespace q4k
