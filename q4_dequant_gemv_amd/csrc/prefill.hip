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
//         acc = fma(-dmin_s, Q_s, fma(d_s, P_s, acc)),   Q_s = sum_j m_j * (sum of x over j),
//     where Q_s is one 16x16x16 MFMA: A holds the eight sub-block sums of each
//     token (divided by 32 so they stay inside the f16 range) as hi + lo f16
//     parts, B the eight six-bit mins (exact).
//
// Data flow.  A preparation kernel writes the activations once per call into
// scratch in the lane order of the MFMA operand (and the sub-block sums).  A
// workgroup of 8 waves owns a 128-row x 128-token tile; each wave 16 rows x
// 128 tokens (8 tiles of 16 x 16), two waves per SIMD.  K is walked in half
// super-blocks: the workgroup copies the next half super-block of activations
// (32 KB) and, every other step, the next super-block of its 128 weight rows
// (18 KB) into LDS with direct-to-LDS buffer loads while the matrix cores work
// on the current one (three buffers of each, one barrier per step).  Every
// output is computed by one lane in a fixed order: results are bitwise
// reproducible.
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
constexpr int kWCopies = kWPieces / 64;
#ifndef Q4K_PREFILL_RT
#define Q4K_PREFILL_RT 1
#endif
#ifndef Q4K_PREFILL_TT
#define Q4K_PREFILL_TT 8
#endif
// waves of a workgroup: RT x TT tiles each cover the 128 x 128 tile
template <int RT, int TT>
constexpr int pf_waves() { return (kPfTile / (16 * RT)) * (kPfTile / (16 * TT)); }

constexpr int kPfRT = Q4K_PREFILL_RT;  // row tiles per wave
constexpr int kPfTT = Q4K_PREFILL_TT;  // token tiles per wave
constexpr int kPfWaves = pf_waves<kPfRT, kPfTT>();
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait for vector memory down to N in flight, nothing else
constexpr int wait_vm(int nvm) { return (nvm & 15) | ((nvm >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVm0 = wait_vm(0);

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
// Each wave owns RT row tiles x TT token tiles of 16 x 16; (128/16/RT) x
// (128/16/TT) waves (4, 8 or 16) cover the 128 x 128 tile.  Building a B
// operand costs about 16 vector instructions per 8 weights and each is used
// TT times; each A operand is read from LDS by every wave with those tokens
// and used RT times.  RT = 1, TT = 8 builds every B operand once per workgroup
// and gives two waves per SIMD (160 registers each), so one wave's operand
// building overlaps the other's matrix-core work: 12-16 % faster than four
// waves of RT = 2 at 512 and 2048 tokens, although each activation fragment
// is read from LDS twice as often.  With ksplit > 1 the workgroup covers super-blocks
// [ks*nsb/ksplit, (ks+1)*nsb/ksplit) and writes its f32 partial tile to
// part[ks] instead of y (added up in a fixed order by prefill_reduce_kernel).
template <int V>
using ic = std::integral_constant<int, V>;

template <typename YT, int RT, int TT>
__global__ __launch_bounds__((64 * pf_waves<RT, TT>()), 1) void prefill_mfma_kernel(const uint8_t *__restrict__ w,
                                                              const uint8_t *__restrict__ xa,
                                                              const uint8_t *__restrict__ xs, YT *__restrict__ y,
                                                              float *__restrict__ part, int64_t m, int64_t n,
                                                              int64_t k, int64_t row_bytes, int nblocks, int nrb,
                                                              int ksplit) {
    constexpr int WR = kPfTile / (16 * RT);  // waves along the rows
    constexpr int NW = pf_waves<RT, TT>();
    static_assert(NW == 4 || NW == 8 || NW == 16, "4, 8 or 16 waves cover the tile");
    constexpr int kAPer = (kAStage / 1024) / NW;      // activation copies per wave per step
    constexpr int kWPer = (kWCopies + NW - 1) / NW;   // weight copies per wave per super-block
    // Three buffers each for the activations (one per step, copied two steps
    // ahead) and the weights (one per super-block, copied one super-block
    // ahead).  Every buffer is its own array and every access names it at
    // compile time (the super-block loop is unrolled by three), so the
    // compiler can tell a copy in flight into one buffer from reads of
    // another and adds no waits of its own.
    __shared__ __align__(16) uint8_t a0[kAStage], a1[kAStage], a2[kAStage];
    __shared__ __align__(16) uint8_t w0[kWStage], w1[kWStage], w2[kWStage];
    // where the copies past the 18 of a super-block land (read by nobody)
    __shared__ __align__(16) uint8_t wpad[1024];
    uint8_t *const abuf[3] = {a0, a1, a2};
    uint8_t *const wbuf[3] = {w0, w1, w2};
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int wr = wave % WR;  // the wave's rows of the tile: 16*RT from 16*RT*wr
    const int wt = wave / WR;  // the wave's tokens: 16*TT from 16*TT*wt
    const int col = lane & 15;
    const int kb = lane >> 4;

    const int rbk = static_cast<int>(blockIdx.x % nrb);
    const int tbk = static_cast<int>((blockIdx.x / nrb) % nblocks);
    const int ks = static_cast<int>(blockIdx.x / (static_cast<int64_t>(nrb) * nblocks));
    const int64_t row0 = static_cast<int64_t>(rbk) * kPfTile;
    const int64_t tok0 = static_cast<int64_t>(tbk) * kPfTile;
    const int nsb_all = static_cast<int>(k / kBlockWeights);
    const int sb_begin = static_cast<int>(static_cast<int64_t>(nsb_all) * ks / ksplit);
    const int nsb = static_cast<int>(static_cast<int64_t>(nsb_all) * (ks + 1) / ksplit) - sb_begin;
    const int64_t rows_here = n - row0 < kPfTile ? n - row0 : kPfTile;
    // rows past n read as zeros; their results are not stored
    const __amdgpu_buffer_rsrc_t wrs = stream_rsrc(w + row0 * row_bytes, static_cast<int>(rows_here * row_bytes));

    // Direct-to-LDS copies: each instruction moves 64 x 16 bytes to LDS base
    // + 16 * lane.  h, s count steps and super-blocks from sb_begin.
    // Copies past the end of the range go through a 0-byte descriptor (or
    // read rows of the next range): they fill buffers nobody reads, and every
    // step issues the same number of copies, so every wait is a constant.
    auto dma_a = [&](int h, uint8_t *dst) {
        const __amdgpu_buffer_rsrc_t ar = stream_rsrc(
            xa + (static_cast<int64_t>(2 * sb_begin + h) * nblocks + tbk) * kAStage, h < 2 * nsb ? kAStage : 0);
        lds_u8 *base = (lds_u8 *)dst;  // generic -> LDS address space
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = wave * kAPer + i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ar, reinterpret_cast<lds_void *>(base + c * 1024), 16,
                                                     c * 1024 + lane * 16, 0, 0, 0);
        }
    };
    auto dma_w = [&](int s, uint8_t *dst) {
        lds_u8 *base = (lds_u8 *)dst;
        // 18 copies of 64 x 16 bytes per super-block, kWPer per wave: the
        // ones past the 18th read past the descriptor (zeros) into wpad
#pragma unroll
        for (int i = 0; i < kWPer; ++i) {
            const int ii = wave + NW * i;
            const int p = ii * 64 + lane;
            const int row = p / 9;
            const int pc = p % 9;
            const uint32_t off = ii < kWPieces / 64 && s < nsb
                                     ? static_cast<uint32_t>(row * row_bytes) +
                                           static_cast<uint32_t>(sb_begin + s) * kBlockBytes +
                                           static_cast<uint32_t>(pc * 16)
                                     : 0x80000000u;
            lds_u8 *dst_c = ii < kWCopies ? base + ii * 1024 : (lds_u8 *)wpad;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, reinterpret_cast<lds_void *>(dst_c), 16, off, 0, 0, 0);
        }
    };
    // a barrier without a memory fence: the waits before it are explicit
    auto barrier = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    float4_t acc[RT][TT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) acc[rt][tt] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const half8_t k1024 = {1024, 1024, 1024, 1024, 1024, 1024, 1024, 1024};

    // One super-block; S3 = s % 3 names the buffers: weights wbuf[S3],
    // activations of its two steps abuf[(2 S3) % 3] and abuf[(2 S3 + 1) % 3].
    // Each step ends by issuing the copies for later steps (after all of its
    // own LDS reads): the activations two steps ahead, and after the second
    // step the weights two super-blocks ahead.
    auto super_block = [&](auto S3c, int s) {
        constexpr int S3 = decltype(S3c)::value;
        const uint8_t *wl = wbuf[S3];
        // the wave's tokens' sub-block sums (A of the min-term product),
        // issued before this super-block's copies so that the waits below
        // cover them
        half4_t qa[TT];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            qa[tt] = *reinterpret_cast<const half4_t *>(
                xs + (static_cast<int64_t>(sb_begin + s) * nblocks + tbk) * kMinBlock + ((wt * TT + tt) * 64 + lane) * 8);
        }
        // headers of the wave's rows: d, dmin, the eight scales (as packed
        // 16-bit pairs) and the mins as the B operand of the min-term product
        // (k-group kb: sub-blocks 4*(kb&1) .. +3)
        float dd[RT], dm[RT];
        uint32_t sc2[RT][8];
        half4_t qb[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const uint4 hdr = *reinterpret_cast<const uint4 *>(wl + (wr * 16 * RT + rt * 16 + col) * kBlockBytes);
            dd[rt] = half_bits_to_float(hdr.x);
            dm[rt] = 32.0f * half_bits_to_float(hdr.x >> 16);  // the sums are stored / 32
            half4_t mv;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                int sc, mm;
                scale_min(hdr.y, hdr.z, hdr.w, q, sc, mm);
                sc2[rt][q] = static_cast<uint32_t>(sc) * 0x00010001u;
                const _Float16 mh = static_cast<_Float16>(static_cast<float>(mm));
                if (q < 4) mv[q] = mh;
                else mv[q - 4] = (kb & 1) ? mh : mv[q - 4];
            }
            qb[rt] = mv;
        }

        float4_t P[RT][TT];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            constexpr int kCur[2] = {(2 * S3) % 3, (2 * S3 + 1) % 3};
            constexpr int kAhead[2] = {(2 * S3 + 2) % 3, (2 * S3 + 3) % 3};
            const int h = 2 * s + half;
            const uint8_t *al = abuf[kCur[half]];
            uint2 codes[RT];
#pragma unroll
            for (int sp = 0; sp < 4; ++sp) {
                const int j = 4 * half + sp;  // sub-block of the super-block
                half8_t a[TT];
#pragma unroll
                for (int tt = 0; tt < TT; ++tt)
                    a[tt] = *reinterpret_cast<const half8_t *>(al + (((wt * TT + tt) * 4 + sp) * 64 + lane) * 16);
                if ((sp & 1) == 0) {
                    // 8 code bytes of group j/2 for this lane's k-group
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        codes[rt] = *reinterpret_cast<const uint2 *>(wl + (wr * 16 * RT + rt * 16 + col) * kBlockBytes +
                                                                     16 + 32 * (j >> 1) + 8 * kb);
                }
                const int shn = (sp & 1) ? 4 : 0;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const uint32_t v0 = pair_operand((codes[rt].x >> shn) & 0x000f000fu, sc2[rt][j]);
                    const uint32_t v1 = pair_operand((codes[rt].x >> (8 + shn)) & 0x000f000fu, sc2[rt][j]);
                    const uint32_t v2 = pair_operand((codes[rt].y >> shn) & 0x000f000fu, sc2[rt][j]);
                    const uint32_t v3 = pair_operand((codes[rt].y >> (8 + shn)) & 0x000f000fu, sc2[rt][j]);
                    const half8_t b = as_half8(u32x4_t{v0, v1, v2, v3}) - k1024;  // sc*q, exact
#pragma unroll
                    for (int tt = 0; tt < TT; ++tt)
                        P[rt][tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[tt], b, j == 0 ? zero : P[rt][tt], 0, 0, 0);
                }
            }
            dma_a(h + 2, abuf[kAhead[half]]);
            if (half == 1) dma_w(s + 2, wbuf[(S3 + 2) % 3]);
            // Copies land in issue order.  At the end of the first step the
            // next step's activations (issued at the end of the previous step)
            // must have landed; after them came this super-block's min-term
            // loads (TT) and the activations two steps ahead (8).  At the end
            // of the second step the activations of the next step (issued at
            // the end of the first) must have landed, and with them the
            // min-term loads and the next super-block's weights (issued a
            // super-block ago); after them only this step's copies (8 + 5).
            if (half == 0) {
                __builtin_amdgcn_s_waitcnt(wait_vm(TT + kAPer));
            } else {
                __builtin_amdgcn_s_waitcnt(wait_vm(kAPer + kWPer));
                // finish super-block s: acc = fma(-dmin, Q, fma(d, P, acc))
#pragma unroll
                for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const float4_t q = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[tt], qb[rt], zero, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            acc[rt][tt][r] = fmaf(-dm[rt], q[r], fmaf(dd[rt], P[rt][tt][r], acc[rt][tt][r]));
                    }
                }
            }
            barrier();
        }
    };

    dma_w(0, w0);
    dma_w(1, w1);
    dma_a(0, a0);
    dma_a(1, a1);
    // step 0's activations and super-block 0's weights have landed (step 1's
    // activations may still fly)
    __builtin_amdgcn_s_waitcnt(wait_vm(kAPer));
    barrier();
    for (int s = 0; s < nsb; s += 3) {
        super_block(ic<0>{}, s);
        if (s + 1 < nsb) super_block(ic<1>{}, s + 1);
        if (s + 2 < nsb) super_block(ic<2>{}, s + 2);
    }
    // no copy may still be writing LDS when the workgroup ends
    __builtin_amdgcn_s_waitcnt(kWaitVm0);

    // lane: row col of each row tile, tokens 4*kb .. 4*kb+3 of each token tile
    float *pk = part + static_cast<int64_t>(ks) * m * n;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int64_t row = row0 + wr * 16 * RT + rt * 16 + col;
        if (row >= n) continue;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tok = tok0 + wt * 16 * TT + tt * 16 + kb * 4 + r;
                if (tok >= m) continue;
                if (ksplit == 1) y[tok * n + row] = static_cast<YT>(acc[rt][tt][r]);
                else pk[tok * n + row] = acc[rt][tt][r];
            }
        }
    }
}

// y = the K parts added in order (part[0] + part[1] + ...), rounded once to YT.
template <typename YT>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float *__restrict__ part, YT *__restrict__ y,
                                                             int64_t count, int ksplit) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count; i += stride) {
        float v = part[i];
        for (int s = 1; s < ksplit; ++s) v += part[static_cast<int64_t>(s) * count + i];
        y[i] = static_cast<YT>(v);
    }
}

hipError_t launch_prefill(const uint8_t *w, const _Float16 *x, void *y, bool y_f16, int64_t m, int64_t n, int64_t k,
                          Workspace &ws, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (ws.query && k == 0) return hipSuccess;
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
    // Too few tiles to fill the CUs: split K across workgroups (each keeps
    // at least 4 super-blocks), partial tiles added by a second kernel.  One
    // workgroup fits a CU (its LDS), so a launch runs in rounds of one
    // workgroup per CU; the split is the smallest that minimizes rounds per
    // unit of K, ceil(tiles * s / CUs) / s (a last round half full costs a
    // whole one).
    const int64_t tiles = nrb * nblocks;
    const int64_t cus = device_cu_count();
    const int64_t max_split = nsb / 4 > 1 ? nsb / 4 : 1;
    int64_t ksplit = 1;
    for (int64_t s = 2; s <= max_split && tiles * (s - 1) < 4 * cus; ++s) {
        // rounds(s) / s < rounds(ksplit) / ksplit, in integers
        const int64_t r = (tiles * s + cus - 1) / cus;
        const int64_t rb = (tiles * ksplit + cus - 1) / cus;
        if (r * ksplit < rb * s) ksplit = s;
    }
    const int64_t part_bytes = ksplit > 1 ? ksplit * m * n * 4 : 0;
    const int64_t total = xa_bytes + xs_bytes + part_bytes;
    if (ws.query) {
        if (total > ws.need) ws.need = total;
        return hipSuccess;
    }
    uint8_t *scratch = nullptr;
    bool owned = false;
    hipError_t e = ws_acquire(ws, total, stream, &scratch, &owned);
    if (e != hipSuccess) return e;
    uint8_t *xa = scratch;
    uint8_t *xs = scratch + xa_bytes;
    float *part = reinterpret_cast<float *>(scratch + xa_bytes + xs_bytes);
    const int64_t prep_threads = mpad * (k / 8);
    hipLaunchKernelGGL(prefill_prep_kernel, dim3(static_cast<unsigned>((prep_threads + 255) / 256)), dim3(256), 0,
                       stream, x, xa, xs, m, mpad, k);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const dim3 grid(static_cast<unsigned>(tiles * ksplit));
        const int64_t rb = (k / kBlockWeights) * kBlockBytes;
        const int nb = static_cast<int>(nblocks), nr = static_cast<int>(nrb), ksp = static_cast<int>(ksplit);
        if (y_f16) {
            hipLaunchKernelGGL((prefill_mfma_kernel<_Float16, kPfRT, kPfTT>), grid, dim3(64 * kPfWaves), 0, stream, w, xa, xs,
                               static_cast<_Float16 *>(y), part, m, n, k, rb, nb, nr, ksp);
        } else {
            hipLaunchKernelGGL((prefill_mfma_kernel<float, kPfRT, kPfTT>), grid, dim3(64 * kPfWaves), 0, stream, w, xa, xs,
                               static_cast<float *>(y), part, m, n, k, rb, nb, nr, ksp);
        }
        e = hipGetLastError();
        if (e == hipSuccess && ksplit > 1) {
            const int64_t count = m * n;
            const int64_t need = (count + 255) / 256;
            const dim3 rg(static_cast<unsigned>(need < 8192 ? need : 8192));
            if (y_f16) {
                hipLaunchKernelGGL(prefill_reduce_kernel<_Float16>, rg, dim3(256), 0, stream, part,
                                   static_cast<_Float16 *>(y), count, ksp);
            } else {
                hipLaunchKernelGGL(prefill_reduce_kernel<float>, rg, dim3(256), 0, stream, part,
                                   static_cast<float *>(y), count, ksp);
            }
            e = hipGetLastError();
        }
    }
    const hipError_t f = ws_release(scratch, owned, stream);
    return e != hipSuccess ? e : f;
}

}  // namespace q4k
