// Skinny Q4_K GEMM: y[t, r] = sum_c W[r,c] x[t,c] for m >= 2 tokens.
//
// selectQ4KFusedVariant ("@simulatte/doppler 0.1.7 -> 0.1.8",
// matmul-selection.js) picks a fused Q4K kernel by whether M == 1; this file
// is the M > 1 side ("Module qwen3_attention" names a W4A16 batched path).
// A few tokens (launch_gemv_tokens) stay on the streaming GEMV kernels, and
// f16 activations at prefill sizes go to the prefill GEMM; the rest is here.
//
// Once enough tokens share each weight the work is a dense contraction, so
// it runs on the matrix cores (v_mfma_f32_16x16x32_f16: 16 tokens x 16 rows x
// 32 weights per instruction; fewer than 16 tokens leave the other rows of the
// activation operand zero).  Exactness of the operands:
//   * B (weights) holds 1024 + sc*q in f16: exact, since sc*q <= 945 < 1024,
//     and built with one packed 16-bit multiply-add per two codes.  Folding
//     the six-bit scale into the operand lets a whole half super-block (4
//     sub-blocks, 128 weights) accumulate into one f32 tile.
//   * A (activations) holds x * 2^-e as f16 hi + lo parts (e per token and
//     half super-block), so every product is exact and the tile carries about
//     22 bits of each x.
// Per half super-block the f32 tile P is finished as
//     acc += 2^e * (d * (P - 1024 * sum(hi + lo)) - dmin * Q),
// where Q = sum_s m_s * sum_{x in s}(hi + lo) comes from a second, small MFMA
// (mins in B, per-sub-block activation sums in A).  A bf16 operand could not
// hold sc*q exactly (8 significant bits), and a bf16 dequantized weight misses
// the 2e-4 * sum|w x| bound at K = 4096.
//
// The hi/lo split carries about 22 bits relative to the largest |x| of its
// (token, half super-block), not of each activation, and a few outliers far
// above the rest (whose weights may be zero) would leave the others coarse.
// The preparation kernel compares, per (half, token) block, the split's total
// remainder E = sum |x - 2^e (hi + lo)| (each remainder exact in f32) with
// S4, the sum of the block's |x| other than its four largest (through a lower
// bound formed without cancellation, rest_bound_tiers), and flags the
// block if E exceeds 2^-15 times that bound.  A
// workgroup whose range holds a flagged block computes its whole tile in f32
// instead (exact_tile: every weight dequantized on its own, every product
// rounded once), so every activation keeps its full precision.
//
// Data flow (gfx950).  A preparation kernel converts x once per call into
// scratch, already in the lane order of the MFMA operand fragments, so each
// wave reads its activations with fully coalesced 1 KB loads straight into
// registers.  A workgroup owns 16*NT rows and a K range; its W waves split the
// K range between them (no activation byte is read twice inside a workgroup,
// and the main loop has no barrier).  Each wave streams its weights and
// activations one step ahead of the matrix cores.  At the end the waves' f32
// tiles are added in LDS in a fixed order and stored; only when the K range
// is split across workgroups (large m with few rows) are the partial tiles
// added into y with f32 atomics.
#include <float.h>
#include <math.h>

#include <type_traits>

#include "launch.h"
#include "q4k_device.h"

namespace q4k {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 as_uint4(u32x4_t v) { return make_uint4(v.x, v.y, v.z, v.w); }
__device__ __forceinline__ float4_t as_float4(u32x4_t v) { return __builtin_bit_cast(float4_t, v); }

constexpr int kStageK = 128;  // activations per stage: half a super-block

// Scratch block of one (stage, 16-token tile):
//   [0, 8192)     A fragments: [MFMA step i][part: hi, lo][lane][8 f16]
//   [8192, 8448)  per token: f16 hi[4], lo[4] of the four sub-block sums of (hi + lo)
//   [8448, 8512)  per token: f32 sum over the stage of (hi + lo)
//   [8512, 8576)  per token: f32 2^e (0: all zero; NaN: a non-finite input)
constexpr int kSubOff = 8192;
constexpr int kBiasOff = 8448;
constexpr int kEscOff = 8512;
constexpr int kTileStageBytes = 8576;

// After the stage blocks, the scratch holds one flag byte per (half
// super-block, padded token): [k/128][16*mt], 1 if that block needs the f32
// path.  Its size, rounded to 16 bytes.
__host__ __device__ constexpr int64_t flag_bytes(int64_t nst, int mt) { return (nst * 16 * mt + 15) / 16 * 16; }

// Position of in-stage activation kk (0..127) in the operand order: the order
// in which the B operand below consumes the codes.  A lane-quarter kq (lanes
// 16kq..16kq+15) owns code bytes [16kq, 16kq+16) of the half block's 64 code
// bytes: group 2h + kq/2, bytes 16*(kq%2).. of that group.  Its dword d (bytes
// 4d..4d+3) splits into the nibble pairs (byte0, byte2) and (byte1, byte3);
// MFMA step i takes the low (i even) or high (i odd) nibbles of dwords
// 2*(i/2) and 2*(i/2)+1.  Result: kq*32 + i*8 + j, j the slot in the lane's 8.
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

// Maximum of unsigned values over aligned groups of 32 lanes (the pairings of
// lane_group_sum<32>: a permlane16 swap, then DPP inside 16-lane rows).
template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp_u32(uint32_t v) {
    const uint32_t moved = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, true));
    return moved > v ? moved : v;
}

__device__ __forceinline__ uint32_t lane32_max_u32(uint32_t v) {
    const auto s = __builtin_amdgcn_permlane16_swap(v, opaque_copy(v), false, false);
    const uint32_t r0 = s[0];
    const uint32_t r1 = opaque_copy(s[1]);
    v = r0 > r1 ? r0 : r1;
    v = max_dpp_u32<0xb1>(v);   // quad_perm [1,0,3,2]
    v = max_dpp_u32<0x4e>(v);   // quad_perm [2,3,0,1]
    v = max_dpp_u32<0x141>(v);  // row_half_mirror
    v = max_dpp_u32<0x140>(v);  // row_mirror
    return v;
}

// ---- activations, converted once per call ----------------------------------
// One half-wave per (stage, token) of the padded token range 16*mt; each lane
// converts four activations.  Tokens >= m are written as zeros.  The same
// kernel zero-fills nzero words at `zero` (an f32 output that the matrix-core
// kernel then accumulates into, or its counters).  XT: float or _Float16
// activations (widened exactly).
template <typename XT>
__global__ __launch_bounds__(256) void x_prep_kernel(const XT *x, uint8_t *__restrict__ xc,
                                                      uint8_t *__restrict__ flags, uint32_t *__restrict__ zero,
                                                      int m, int mt, int64_t k, int64_t nzero) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    for (int64_t i = gid; i < nzero; i += static_cast<int64_t>(gridDim.x) * 256) zero[i] = 0u;

    const int64_t nst = k / kStageK;
    const int tpad = 16 * mt;
    const int64_t pairs = nst * tpad;
    const int c = threadIdx.x & 31;
    int64_t pair = gid >> 5;
    const bool live = pair < pairs;
    if (!live) pair = pairs - 1;  // keep the half-wave's shuffles uniform; no writes
    const int64_t st = pair / tpad;
    const int tok = static_cast<int>(pair % tpad);
    const bool real = tok < m;
    const XT *px = x + static_cast<int64_t>(real ? tok : 0) * k + st * kStageK + 4 * c;
    // The largest magnitude is taken on the bit patterns of |x|: integer
    // order is numeric order for non-negative floats, and every NaN pattern
    // lies above infinity's, so a NaN counts as non-finite.
    float v[4];
    uint32_t mb = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        v[b] = real ? static_cast<float>(px[b]) : 0.0f;
        const uint32_t a = __float_as_uint(v[b]) & 0x7fffffffu;
        mb = a > mb ? a : mb;
    }
    mb = lane32_max_u32(mb);
    const bool finite = mb < 0x7f800000u;
    const bool nz = finite && mb != 0u;
    const float amax = __uint_as_float(mb);
    const int e = nz ? __builtin_amdgcn_frexp_expf(amax) - 1 : 0;  // ilogb of a finite non-zero amax
    _Float16 hi[4], lo[4];
    float sv[4];
    float part = 0.0f;
    // magnitudes in units of 2^e
    float mag[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        sv[b] = nz ? ldexpf(v[b], -e) : 0.0f;
        hi[b] = static_cast<_Float16>(sv[b]);
        const float rem = sv[b] - static_cast<float>(hi[b]);  // exact in f32
        lo[b] = static_cast<_Float16>(rem);
        mag[b] = fabsf(sv[b]);
        part += static_cast<float>(hi[b]) + static_cast<float>(lo[b]);
    }
    const float sub8 = lane_group_sum<8>(part);
    const float tot = lane_group_sum<32>(part);
    // a lower bound of the magnitude without the four largest: the sum of all
    // minus four times the largest (here 1 <= largest < 2); the total
    // remainder E and the tighter bounds only where that does not clear the
    // test.  |sv - hi| <= 2^-11 and |sv - hi - lo| <= 2^-23, so E <= 128 *
    // 2^-23 = 2^-16 and E * 2^15 <= 1/2: a block whose first bound reaches 1/2
    // passes whatever E is.
    const float abs_sum = lane_group_sum<32>((mag[0] + mag[1]) + (mag[2] + mag[3]));
    const float amax_s = nz ? ldexpf(amax, -e) : 0.0f;
    const float first = abs_sum - 4.0f * amax_s;
    uint8_t flag = 0;
    if (__builtin_amdgcn_ballot_w64(nz && !(first >= 0.5f)) != 0) {
        float round_sum = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float rem = sv[b] - static_cast<float>(hi[b]);
            round_sum += fabsf(rem - static_cast<float>(lo[b]));  // exact: what the split leaves out
        }
        round_sum = lane_group_sum<32>(round_sum);
        const float rest = rest_bound_tiers<32>(mag, first, round_sum * 32768.0f);
        flag = round_sum * 32768.0f > rest ? 1 : 0;
    }
    if (!live) return;
    if (c == 0) flags[st * tpad + tok] = flag;
    uint8_t *blk = xc + (st * mt + tok / 16) * kTileStageBytes;
    const int col = tok & 15;
    // activations 4c..4c+3 land at positions pos + {0, 2, 1, 3} of one lane
    const int pos = stage_pos(4 * c);
    const int kq = pos >> 5;
    const int i = (pos >> 3) & 3;
    const int j0 = pos & 7;
    const int lane_slot = col + 16 * kq;
    *reinterpret_cast<half4_t *>(blk + ((i * 2 + 0) * 64 + lane_slot) * 16 + j0 * 2) =
        half4_t{hi[0], hi[2], hi[1], hi[3]};
    *reinterpret_cast<half4_t *>(blk + ((i * 2 + 1) * 64 + lane_slot) * 16 + j0 * 2) =
        half4_t{lo[0], lo[2], lo[1], lo[3]};
    if ((c & 7) == 0) {
        _Float16 *s = reinterpret_cast<_Float16 *>(blk + kSubOff) + col * 8;
        const _Float16 sh = static_cast<_Float16>(sub8);
        s[c >> 3] = sh;
        s[4 + (c >> 3)] = static_cast<_Float16>(sub8 - static_cast<float>(sh));
    }
    if (c == 0) {
        reinterpret_cast<float *>(blk + kBiasOff)[col] = tot;
        reinterpret_cast<float *>(blk + kEscOff)[col] = finite ? (nz ? ldexpf(1.0f, e) : 0.0f) : NAN;
    }
}

// ---- the f32 path -------------------------------------------------------------
// Rows [row0, row1) of W times tokens [0, m) of x over super-blocks
// [sb0, sb1), in f32 with every weight on its own: w = fma(d*sc, q, -dmin*m)
// (d*sc*q is exact in f32, so this is the correctly rounded weight the
// dequant kernel writes) and every product rounded once.  Wave `wave` of
// `nwaves` takes rows row0 + wave, row0 + wave + nwaves, ...; for each row and
// four tokens at a time, lane l multiplies weights 4l .. 4l+3 of each
// super-block (four products summed in f32), adds them into an f64 sum over
// the super-blocks (any K range without a long chain of f32 roundings), and
// the lane sums are added across the wave.  The results are
// stored (ADD false: y = YT of the sum) or added into f32 y with atomics.  A
// non-finite activation makes its token's results NaN, as on the matrix
// cores: the sum of 0 * x (0 for finite x, NaN otherwise) is added.
template <typename XT, typename YT, bool ADD>
__device__ __attribute__((noinline)) void exact_tile(const uint8_t *__restrict__ w, int64_t row_bytes,
                                                    const XT *__restrict__ x, int64_t k,
                           int m, YT *__restrict__ y, int64_t n, int64_t row0, int64_t row1, int sb0, int sb1,
                           int wave, int nwaves) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;             // 64-weight group of the lane's four weights
    const int r = 4 * (lane & 15);       // their place inside the group
    const int j = 2 * g + (r >> 5);      // sub-block
    const int shift = r >= 32 ? 4 : 0;   // high nibbles for the second sub-block of the group
    const int code_off = 16 + 32 * g + (r & 31);
    for (int64_t row = row0 + wave; row < row1; row += nwaves) {
        const uint8_t *wr = w + row * row_bytes;
        for (int t0 = 0; t0 < m; t0 += 4) {
            double acc[4] = {0.0, 0.0, 0.0, 0.0};
            float nf[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int sb = sb0; sb < sb1; ++sb) {
                const uint8_t *blk = wr + static_cast<int64_t>(sb) * kBlockBytes;
                const uint4 hdr = *reinterpret_cast<const uint4 *>(blk);
                const uint32_t q4 = (*reinterpret_cast<const uint32_t *>(blk + code_off) >> shift) & 0x0f0f0f0fu;
                int sc, mn;
                scale_min(hdr.y, hdr.z, hdr.w, j, sc, mn);
                const float dl = half_bits_to_float(hdr.x) * static_cast<float>(sc);
                const float ml = half_bits_to_float(hdr.x >> 16) * static_cast<float>(mn);
                float wv[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) wv[b] = fmaf(dl, static_cast<float>((q4 >> (8 * b)) & 0xffu), -ml);
                const int64_t col = static_cast<int64_t>(sb) * kBlockWeights + 4 * lane;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if (t0 + u < m) {
                        const XT *xp = x + static_cast<int64_t>(t0 + u) * k + col;
                        float part = 0.0f;
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            const float xv = static_cast<float>(xp[b]);
                            part = fmaf(wv[b], xv, part);
                            nf[u] = fmaf(xv, 0.0f, nf[u]);
                        }
                        acc[u] += static_cast<double>(part);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float v = lane_group_sum<64>(static_cast<float>(acc[u]) + nf[u]);
                if (lane == 0 && t0 + u < m) {
                    YT *dst = y + static_cast<int64_t>(t0 + u) * n + row;
                    if constexpr (ADD) unsafeAtomicAdd(dst, v);
                    else *dst = static_cast<YT>(v);
                }
            }
        }
    }
}

// The OR of this thread's share of the flag bytes [off, off + count) of the
// scratch (whole dwords: off and count are multiples of 16).  Issued before
// a kernel's first weight loads, so that waiting for it (in issue order)
// leaves those loads in flight.
__device__ __forceinline__ uint32_t load_flags(__amdgpu_buffer_rsrc_t ar, int64_t off, int64_t count) {
    uint32_t any = 0;
    for (int64_t i = 4 * static_cast<int64_t>(threadIdx.x); i < count; i += 4 * static_cast<int64_t>(blockDim.x))
        any |= __builtin_amdgcn_raw_buffer_load_b32(ar, static_cast<int>(off + i), 0, 0);
    return any;
}

// Whether any wave of the workgroup saw a set flag: each wave's lane 0 writes
// its ballot to wflag[wave], then a barrier.  The barrier is bare (no fence),
// with only the LDS write waited for, so weight loads in flight stay in
// flight.
__device__ __forceinline__ bool workgroup_any(uint32_t any, int *wflag, int nw) {
    const bool wave_any = __builtin_amdgcn_ballot_w64(any != 0) != 0;
    if ((threadIdx.x & 63) == 0) wflag[threadIdx.x >> 6] = wave_any ? 1 : 0;
    // lgkmcnt(0) only (vmcnt and expcnt at their maxima, gfx9 encoding)
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    int all = 0;
    for (int v = 0; v < nw; ++v) all |= wflag[v];
    return all != 0;
}

// ---- the matrix-core kernel ---------------------------------------------------
// Activations of one (half super-block, token tile) step.
struct AStep {
    uint4 f[8];     // fragments: [MFMA step i][hi, lo]
    uint4 sub;      // the lane's token: f16 hi[4], lo[4] sub-block sums
    float4_t bias;  // tokens 4kq .. 4kq+3 of the tile
    float4_t esc;
};

// B operands of one row tile for one half super-block.
struct BOps {
    half8_t b[4];
    half8_t bmin;
    float d, dmin;
};

// B operands of half hw of a super-block for the lane's row (col) and
// k-quarter kq, from the super-block's 16-byte header and the quarter's 16
// code bytes; ps = pair_select(2 * hw + kq / 2).
__device__ __forceinline__ void build_b_ops(BOps &o, uint4 hdr, uint4 qv, const PairSelect &ps, int kq) {
    o.d = half_bits_to_float(hdr.x);
    o.dmin = half_bits_to_float(hdr.x >> 16);
    uint32_t scp, mp;
    scale_min_pair(hdr.y, hdr.z, hdr.w, ps, scp, mp);
    const uint32_t sc2_lo = (scp & 0xffu) * 0x00010001u;
    const uint32_t sc2_hi = ((scp >> 8) & 0xffu) * 0x00010001u;
    const uint32_t u[4] = {qv.x, qv.y, qv.z, qv.w};
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
        o.b[i] = __builtin_bit_cast(half8_t, u32x4_t{v4[0], v4[1], v4[2], v4[3]});
    }
    // mins of the quarter's two sub-blocks (even quarters only) as exact f16
    const _Float16 m0 = (kq & 1) ? _Float16(0) : static_cast<_Float16>(static_cast<float>(mp & 0xffu));
    const _Float16 m1 = (kq & 1) ? _Float16(0) : static_cast<_Float16>(static_cast<float>((mp >> 8) & 0xffu));
    o.bmin = half8_t{m0, m1, 0, 0, 0, 0, 0, 0};
}

// One (row tile, token tile) product of a half super-block and its epilogue:
// out[r] += 2^e * (d * (P - 1024 * sum(hi + lo)) - dmin * Q) for the lane's
// tokens 4*kq + r.  TWO_CHAINS: the hi and lo products accumulate into two
// independent tiles, added at the end, so consecutive matrix-core
// instructions do not wait on each other (faster when a wave has many
// token tiles to multiply; one chain is as fast otherwise).
template <bool TWO_CHAINS = false>
__device__ __forceinline__ void mfma_half(const BOps &bo, const AStep &a, float4_t &out, int kq) {
    // the lane's token's sums of its quarter's two sub-blocks, hi and lo
    const int gg = kq >> 1;
    const uint32_t shi = (kq & 1) ? 0u : (gg ? a.sub.y : a.sub.x);
    const uint32_t slo = (kq & 1) ? 0u : (gg ? a.sub.w : a.sub.z);
    const half8_t amin_hi = __builtin_bit_cast(half8_t, u32x4_t{shi, 0u, 0u, 0u});
    const half8_t amin_lo = __builtin_bit_cast(half8_t, u32x4_t{slo, 0u, 0u, 0u});
    float4_t pacc = {0.0f, 0.0f, 0.0f, 0.0f};
    float4_t lacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a.f[2 * i]), bo.b[i], pacc, 0, 0, 0);
        float4_t &second = TWO_CHAINS ? lacc : pacc;
        second =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a.f[2 * i + 1]), bo.b[i], second, 0, 0, 0);
    }
    if constexpr (TWO_CHAINS) pacc += lacc;
    float4_t qacc = {0.0f, 0.0f, 0.0f, 0.0f};
    qacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(amin_hi, bo.bmin, qacc, 0, 0, 0);
    qacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(amin_lo, bo.bmin, qacc, 0, 0, 0);
    // pacc[r] = sum_k A[tok_r, k] * (1024 + sc q)[k, row]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float code_part = pacc[r] - 1024.0f * a.bias[r];
        out[r] += a.esc[r] * (bo.d * code_part - bo.dmin * qacc[r]);
    }
}

// Workgroup = W = 2S waves, 16*NT rows, a K range [sb0, sb1) of super-blocks
// (block b: row block b / ksplit, K part b % ksplit).  The range is walked in
// stages of S super-blocks.  Each stage's weights (16*NT rows x 144*S bytes)
// are copied into LDS with loads that run along the rows (consecutive lanes,
// consecutive 16-byte pieces of a row: long runs of each row, as the weights
// are laid out), P stages ahead of use, into a double-buffered LDS stage;
// one barrier per stage.  Wave w multiplies half super-block w of the stage
// for all row and token tiles, with its activations read from scratch into
// registers one step ahead.  At the end the waves' sums are added in LDS in a
// fixed order, then stored (ksplit == 1) or added into y with atomics
// (ksplit > 1, y zeroed first).
// Stages of weights in flight.  Two: more only deepens the burst of loads
// every workgroup issues at the start (the first stage then lands later) and
// takes registers from the operands.
template <int MT>
constexpr int weight_stages_ahead() { return 2; }

template <int NT, int S>
struct StageGeom {
    static constexpr int kRows = 16 * NT;
    static constexpr int kRowLds = 144 * S + 16;  // padded: the 16 rows of a tile hit distinct LDS banks
    static constexpr int kChunks = kRows * 9 * S;  // 16-byte pieces per stage
    static constexpr int kBlock = 128 * S;
    static constexpr int kLoads = (kChunks + kBlock - 1) / kBlock;  // per thread per stage
    static constexpr int kStageLds = kRows * kRowLds;
};

// YT: float or _Float16 output (f16 only with ksplit == 1: the atomics add f32).
// x: the activations themselves (the f32 path's input); the flag bytes start
// at flag_off in xc.
template <int NT, int MT, int S, typename YT, typename XT>
__global__ __launch_bounds__(128 * S, 1) void batched_mfma_kernel(const uint8_t *__restrict__ w,
                                                                  const uint8_t *__restrict__ xc,
                                                                  YT *__restrict__ y, int m, int64_t n,
                                                                  int64_t k, int64_t row_bytes, int ksplit,
                                                                  int64_t xc_bytes, const XT *__restrict__ x,
                                                                  int64_t flag_off) {
    using G = StageGeom<NT, S>;
    constexpr int W = 2 * S;
    constexpr int P = weight_stages_ahead<MT>();
    __shared__ __align__(16) uint8_t stage_lds[2][G::kStageLds];
    __shared__ __align__(16) float4_t red[W][NT * MT][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int col = lane & 15;
    const int kq = lane >> 4;

    const int nsb = static_cast<int>(k / kBlockWeights);
    const int64_t rb = blockIdx.x / ksplit;
    const int ks = static_cast<int>(blockIdx.x % ksplit);
    const int sb0 = static_cast<int>(static_cast<int64_t>(nsb) * ks / ksplit);
    const int sb1 = static_cast<int>(static_cast<int64_t>(nsb) * (ks + 1) / ksplit);
    const int nstages = (sb1 - sb0 + S - 1) / S;

    const int64_t row0 = rb * G::kRows;
    const int64_t rows_here = n - row0 < G::kRows ? n - row0 : G::kRows;
    // rows past n read as zeros; their results are not stored
    const __amdgpu_buffer_rsrc_t wr = stream_rsrc(w + row0 * row_bytes, static_cast<int>(rows_here * row_bytes));
    const __amdgpu_buffer_rsrc_t ar = stream_rsrc(xc, static_cast<int>(xc_bytes));
    // flags of this workgroup's halves, all token tiles: loaded first
    const uint32_t flag_bits = load_flags(ar, flag_off + 2 * static_cast<int64_t>(sb0) * 16 * MT,
                                          2 * static_cast<int64_t>(sb1 - sb0) * 16 * MT);

    // ---- this thread's pieces of every stage copy
    uint32_t g_off[G::kLoads];   // byte offset in the row block, stage base excluded
    uint32_t l_off[G::kLoads];   // byte offset in the LDS stage
    int p_sb[G::kLoads];         // super-block of the piece inside the stage (S: padding)
#pragma unroll
    for (int j = 0; j < G::kLoads; ++j) {
        const int c = j * G::kBlock + static_cast<int>(threadIdx.x);
        const bool ok = c < G::kChunks;
        const int cc = ok ? c : 0;
        const int row = cc / (9 * S);
        const int piece = cc % (9 * S);
        g_off[j] = static_cast<uint32_t>(row * row_bytes + piece * 16);
        l_off[j] = static_cast<uint32_t>(row * G::kRowLds + piece * 16);
        p_sb[j] = ok ? piece / 9 : S;
    }
    typedef uint4 StageRegs[G::kLoads];
    // loads of stage st (nothing past the range: such pieces point past the
    // descriptor's end and read zeros without a fetch)
    auto issue_stage = [&](StageRegs &r, int st) {
        const int sbs = sb0 + st * S;
        const int sbn = sb1 - sbs;  // super-blocks left in the range (may be <= 0)
#pragma unroll
        for (int j = 0; j < G::kLoads; ++j) {
            const uint32_t off = p_sb[j] < sbn ? g_off[j] : 0x40000000u;
            r[j] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(wr, static_cast<int>(off), sbs * kBlockBytes, 0));
        }
    };
    auto write_stage = [&](const StageRegs &r, int buf) {
#pragma unroll
        for (int j = 0; j < G::kLoads; ++j) {
            if (j * G::kBlock + static_cast<int>(threadIdx.x) < G::kChunks)
                *reinterpret_cast<uint4 *>(&stage_lds[buf][l_off[j]]) = r[j];
        }
    };

    // ---- activations: a lane whose token (per tile) is past m reads nothing
    uint32_t a_lane[MT];
#pragma unroll
    for (int p = 0; p < MT; ++p) a_lane[p] = 16 * p + col < m ? 0u : 0x40000000u;
    const int last_half = static_cast<int>(k / kStageK) - 1;
    auto load_a = [&](AStep &a, int h, int p) {
        // past the K range (a prefetch whose results are not used): the last
        // stage, so that every read stays inside the scratch
        const int hc = h < last_half ? h : last_half;
        const int soff = (hc * MT + p) * kTileStageBytes;
#pragma unroll
        for (int f = 0; f < 8; ++f)
            a.f[f] = as_uint4(
                __builtin_amdgcn_raw_buffer_load_b128(ar, static_cast<int>(a_lane[p] + f * 1024 + lane * 16), soff, 0));
        a.sub = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(ar, static_cast<int>(a_lane[p] + kSubOff + col * 16), soff, 0));
        a.bias = as_float4(__builtin_amdgcn_raw_buffer_load_b128(ar, kBiasOff + kq * 16, soff, 0));
        a.esc = as_float4(__builtin_amdgcn_raw_buffer_load_b128(ar, kEscOff + kq * 16, soff, 0));
    };
    // the wave's half super-block of stage st (past the range: the last stage,
    // whose results are not used)
    const int sbl = wave >> 1;   // super-block inside the stage
    const int hw = wave & 1;     // half of that super-block
    auto half_of = [&](int st) { return 2 * (sb0 + st * S + sbl) + hw; };
    auto half_live = [&](int st) { return st < nstages && sb0 + st * S + sbl < sb1; };

    // B operands of row tile t from the LDS stage
    const PairSelect ps = pair_select(2 * hw + (kq >> 1));
    auto build_b = [&](BOps &o, int buf, int t) {
        const uint8_t *rowp = &stage_lds[buf][(16 * t + col) * G::kRowLds + sbl * kBlockBytes];
        const uint4 hdr = *reinterpret_cast<const uint4 *>(rowp);
        const uint4 qv = *reinterpret_cast<const uint4 *>(rowp + 16 + 64 * hw + 16 * kq);
        build_b_ops(o, hdr, qv, ps, kq);
    };

    float4_t acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int p = 0; p < MT; ++p) acc[t][p] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto multiply = [&](const BOps &bo, const AStep &a, float4_t &out) { mfma_half<(MT >= 4)>(bo, a, out, kq); };

    // ---- pipeline: weights P stages ahead (register ring -> LDS), the wave's
    // activations one step ahead.  Unrolled by P so every ring slot, LDS
    // buffer and activation buffer index is a constant.
    static_assert(P % 2 == 0, "LDS buffer parity must repeat with the ring");
    StageRegs ring[P];
    AStep abuf[2];
    BOps bo[MT == 1 ? 1 : NT];
#pragma unroll
    for (int q = 0; q < P; ++q) issue_stage(ring[q], q);
    load_a(abuf[0], half_of(0), 0);
    // a flagged block in the range: the whole tile on the f32 path instead
    {
        __shared__ int wflag[W];
        if (workgroup_any(flag_bits, wflag, W)) {
            if (ksplit == 1) {
                exact_tile<XT, YT, false>(w, row_bytes, x, k, m, y, n, row0, row0 + rows_here, sb0, sb1, wave, W);
            } else if constexpr (std::is_same_v<YT, float>) {
                exact_tile<XT, float, true>(w, row_bytes, x, k, m, y, n, row0, row0 + rows_here, sb0, sb1, wave, W);
            }
            return;
        }
    }
    write_stage(ring[0], 0);
    issue_stage(ring[0], P);
    for (int s0 = 0; s0 < nstages; s0 += P) {
#pragma unroll
        for (int u = 0; u < P; ++u) {
            const int st = s0 + u;
            __syncthreads();  // stage st is in LDS; every wave is done with stage st-1
            if (st >= nstages) break;
            const bool live = half_live(st);
#pragma unroll
            for (int p = 0; p < MT; ++p) {
                const int step = u * MT + p;
                if (p + 1 < MT) load_a(abuf[(step + 1) & 1], half_of(st), p + 1);
                else load_a(abuf[(step + 1) & 1], half_of(st + 1), 0);
                if (live) {
                    if constexpr (MT == 1) {
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            build_b(bo[0], u & 1, t);
                            multiply(bo[0], abuf[step & 1], acc[t][0]);
                        }
                    } else {
                        if (p == 0) {
#pragma unroll
                            for (int t = 0; t < NT; ++t) build_b(bo[t], u & 1, t);
                        }
#pragma unroll
                        for (int t = 0; t < NT; ++t) multiply(bo[t], abuf[step & 1], acc[t][p]);
                    }
                }
            }
            // stage st+1 into the other LDS buffer (its loads were issued P-1
            // stages ago), then reuse the ring slot for stage st+1+P
            write_stage(ring[(u + 1) % P], (u + 1) & 1);
            issue_stage(ring[(u + 1) % P], st + 1 + P);
        }
    }

    // add the W waves' tiles in wave order, then store or accumulate
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int p = 0; p < MT; ++p) red[wave][t * MT + p][lane] = acc[t][p];
    __syncthreads();
    for (int e = static_cast<int>(threadIdx.x); e < NT * MT * 64; e += G::kBlock) {
        const int tp = e >> 6;
        const int ln = e & 63;
        float4_t sum = red[0][tp][ln];
#pragma unroll
        for (int v = 1; v < W; ++v) sum += red[v][tp][ln];
        const int t = tp / MT;
        const int p = tp % MT;
        const int64_t row = row0 + 16 * t + (ln & 15);
        if (row >= n) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = 16 * p + 4 * (ln >> 4) + r;
            if (tok >= m) continue;
            YT *dst = y + static_cast<int64_t>(tok) * n + row;
            if constexpr (std::is_same_v<YT, float>) {
                if (ksplit == 1) *dst = sum[r];
                else unsafeAtomicAdd(dst, sum[r]);
            } else {
                *dst = static_cast<YT>(sum[r]);
            }
        }
    }
}

// ---- up to 16 tokens, K <= 4096: a weight stream into the matrix cores ------
// Wave w of the workgroup owns half super-blocks [H*w, H*w + H) of every row
// and keeps their activation fragments (one 16-token tile, from the
// preparation kernel's scratch) in registers for the whole call, and their
// per-token sums and scales in LDS (read per tile).  The
// workgroup streams 16-row tiles (tile blockIdx.x + c*gridDim.x); each wave
// loads its part of a tile straight into registers, NB - 1 tiles ahead of the
// one it multiplies (per lane: row `col`'s super-block headers and 16 code
// bytes per half), builds the B operands and runs the same half super-block
// products as the staged kernel.  Each wave's tile sums go to LDS; every
// kStreamFlush tiles, after a barrier, one thread per (tile, lane) adds the
// waves' sums in wave order and stores them, so the result does not depend on
// timing.  Halves past the row (the half count not a multiple of H) are
// skipped.
constexpr int kStreamFlush = 2;
constexpr int kStreamMaxWaves = 16;
constexpr int kStreamMaxHalves = 32;
constexpr int64_t kStreamMaxK = kStreamMaxHalves * kStageK;
// Waves per workgroup at most: 16 with one or two halves per wave (128
// registers each), 8 with four (256 registers: two waves per SIMD).
template <int H>
constexpr int stream_max_waves() { return H <= 2 ? 16 : 8; }

template <int H, int NB, typename YT, typename XT, int KP = 1>
__global__ __launch_bounds__(64 * (KP == 1 ? stream_max_waves<H>() : 8), 1) void stream_mfma_kernel(
    const uint8_t *__restrict__ w, const uint8_t *__restrict__ xc, YT *__restrict__ y, int m, int64_t n, int64_t k,
    int64_t row_bytes, int64_t xc_bytes, const XT *__restrict__ x, int64_t flag_off) {
    static_assert(H == 1 || H == 2 || H == 4, "a wave's halves start a super-block (H even) or are one half");
    static_assert(KP == 1 || (KP == 2 && std::is_same_v<YT, float>), "K parts add f32 partial tiles");
    constexpr int NH = (H + 1) / 2;  // super-blocks (headers) per wave
    __shared__ __align__(16) float4_t part[2][kStreamFlush][stream_max_waves<H>()][64];
    // per half: the scratch block's tail from kSubOff (sub-block sums, bias,
    // 2^e), 24 pieces of 16 bytes
    constexpr int kTail = (kTileStageBytes - kSubOff) / 16;
    __shared__ __align__(16) uint4 tails[kStreamMaxHalves][kTail];
    const int nw = static_cast<int>(blockDim.x) >> 6;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int nhalf = static_cast<int>(k / kStageK);
    // KP = 2: workgroup b takes K part b % 2 (half the halves) of the tiles
    // b / 2, b / 2 + gridDim.x / 2, ...; its partial tiles are added into y
    // (zeroed by the preparation kernel), two addends per output
    const int kp = KP == 1 ? 0 : static_cast<int>(blockIdx.x % KP);
    const int tblk = static_cast<int>(blockIdx.x / KP);
    const int tgrid = static_cast<int>(gridDim.x / KP);
    const int hw0 = kp * (nhalf / KP) + wave * H;  // the wave's first half (even when H >= 2)
    const int sb = hw0 >> 1;   // its first super-block

    // activations of the wave's halves (a lane whose token is past m reads
    // zeros; a half past the row reads the last one and is skipped); the
    // flags of every half first
    const __amdgpu_buffer_rsrc_t ar = stream_rsrc(xc, static_cast<int>(xc_bytes));
    const uint32_t flag_bits = load_flags(ar, flag_off, static_cast<int64_t>(nhalf) * 16);
    const uint32_t a_off = col < m ? 0u : 0x40000000u;
    uint4 af[H][8];
    PairSelect ps[H];
    int hl[H];  // the half's row of `tails`
#pragma unroll
    for (int h = 0; h < H; ++h) {
        hl[h] = hw0 + h < nhalf ? hw0 + h : nhalf - 1;
        const int soff = hl[h] * kTileStageBytes;
#pragma unroll
        for (int f = 0; f < 8; ++f)
            af[h][f] = as_uint4(
                __builtin_amdgcn_raw_buffer_load_b128(ar, static_cast<int>(a_off + f * 1024 + lane * 16), soff, 0));
        if (lane < kTail) tails[hl[h]][lane] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(ar, kSubOff + lane * 16, soff, 0));
        ps[h] = pair_select(2 * ((hw0 + h) & 1) + (kq >> 1));
    }
    __shared__ int wflag[stream_max_waves<H>()];
    const bool exact = workgroup_any(flag_bits, wflag, nw);
    __syncthreads();

    // the host keeps gridDim.x / KP <= the number of tiles: every workgroup has one
    const int64_t ntiles = (n + 15) / 16;
    const int my_tiles = static_cast<int>((ntiles - 1 - tblk) / tgrid) + 1;
    auto tile_row0 = [&](int c) -> int64_t {
        return (static_cast<int64_t>(tblk) + static_cast<int64_t>(c) * tgrid) * 16;
    };
    if (exact) {
        // a flagged block: the workgroup's tiles (its K part) on the f32 path
        const int nsb = static_cast<int>(k / kBlockWeights);
        for (int c = 0; c < my_tiles; ++c) {
            const int64_t r0 = tile_row0(c);
            const int64_t r1 = r0 + 16 < n ? r0 + 16 : n;
            if constexpr (KP == 1) {
                exact_tile<XT, YT, false>(w, row_bytes, x, k, m, y, n, r0, r1, 0, nsb, wave, nw);
            } else {
                exact_tile<XT, float, true>(w, row_bytes, x, k, m, y, n, r0, r1, kp * nsb / KP, (kp + 1) * nsb / KP,
                                            wave, nw);
            }
        }
        return;
    }
    // byte offset of the lane's header inside a tile (< 16 * 2304 + 2304)
    const uint32_t lane_off = static_cast<uint32_t>(col * row_bytes + sb * kBlockBytes);
    struct TileLoads {
        uint4 hdr[NH];
        uint4 q[H];
    };
    // loads of tile c of this workgroup (none past the last: a 0-byte
    // descriptor, so the loads read zeros without a fetch)
    auto issue = [&](TileLoads &L, int c) {
        const bool live = c < my_tiles;
        const int64_t row0 = live ? tile_row0(c) : 0;
        const int64_t rows = n - row0 < 16 ? n - row0 : 16;
        const int nrec = __builtin_amdgcn_readfirstlane(live ? static_cast<int>(rows * row_bytes) : 0);
        const uint8_t *base = reinterpret_cast<const uint8_t *>(wave_uniform(reinterpret_cast<int64_t>(w + row0 * row_bytes)));
        const __amdgpu_buffer_rsrc_t r = stream_rsrc(base, nrec);
#pragma unroll
        for (int j = 0; j < NH; ++j) L.hdr[j] = buffer_load16(r, lane_off + j * kBlockBytes);
#pragma unroll
        for (int h = 0; h < H; ++h) {
            L.q[h] = buffer_load16(r, lane_off + (h >> 1) * kBlockBytes + 16u + 64u * ((hw0 + h) & 1) + 16u * kq);
        }
    };

    TileLoads ring[NB];
#pragma unroll
    for (int b = 0; b + 1 < NB; ++b) issue(ring[b], b);
    for (int c = 0; c < my_tiles; c += NB) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int cur = c + u;
            issue(ring[(u + NB - 1) % NB], cur + NB - 1);
            float4_t out = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int h = 0; h < H; ++h) {
                if (H == 1 || hw0 + h < nhalf) {
                    AStep a;
#pragma unroll
                    for (int f = 0; f < 8; ++f) a.f[f] = af[h][f];
                    a.sub = tails[hl[h]][col];
                    a.bias = __builtin_bit_cast(float4_t, tails[hl[h]][(kBiasOff - kSubOff) / 16 + kq]);
                    a.esc = __builtin_bit_cast(float4_t, tails[hl[h]][(kEscOff - kSubOff) / 16 + kq]);
                    BOps bo;
                    build_b_ops(bo, ring[u].hdr[h >> 1], ring[u].q[h], ps[h], kq);
                    mfma_half(bo, a, out, kq);
                }
            }
            const int d = cur % kStreamFlush;
            const int half = (cur / kStreamFlush) & 1;
            part[half][d][wave][lane] = out;
            if (d == kStreamFlush - 1 || cur + 1 == my_tiles) {
                __syncthreads();
                const int t = static_cast<int>(threadIdx.x);
                if (t < (d + 1) * 64) {
                    const int dd = t >> 6;
                    const int ln = t & 63;
                    float4_t sum = part[half][dd][0][ln];
                    for (int v = 1; v < nw; ++v) sum += part[half][dd][v][ln];
                    const int64_t row = tile_row0(cur - d + dd) + (ln & 15);
                    if (row < n) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tok = 4 * (ln >> 4) + r;
                            if (tok >= m) continue;
                            YT *dst = y + static_cast<int64_t>(tok) * n + row;
                            if constexpr (KP == 1) *dst = static_cast<YT>(sum[r]);
                            else unsafeAtomicAdd(dst, sum[r]);
                        }
                    }
                }
            }
            if (cur + 1 >= my_tiles) break;
        }
    }
}

// ---- the same, K split in two, with the weights staged through LDS ----------
// At K = 4096 with few tiles per CU (the two-part form above), each wave's
// share of a tile is 16 rows x one super-block: 16 runs of 144 bytes.  Three
// loads per wave copy them straight into LDS ([row][144 bytes], lane l of
// load i taking 16-byte piece 64 i + l), so a ring of D tiles per wave costs
// no registers and D tiles' weights are in flight from the start, where the
// register ring held one.  D = 2: deeper rings put more of every
// workgroup's loads into one burst at the start, which delays each first
// tile (9B gate, 16 tokens, per call with the preparation: 13.4 / 13.9 /
// 14.6 us for D = 2 / 3 / 4, the register ring 15.0).  A wave reads only its own ring
// slots, so it waits for its own loads alone (wait_vm) and needs no barrier
// for them; the barriers of the sums between waves wait for LDS operations
// only, so the stream keeps running across them.  Everything else (the
// activation fragments in registers, the B operands, the products, the fixed
// order of the sums, two addends per output in y) is the kernel above with
// H = 2, K parts = 2.
#ifndef Q4K_STREAM_LDS
#define Q4K_STREAM_LDS 1
#endif
#ifndef Q4K_STREAM_LDS_D
#define Q4K_STREAM_LDS_D 2
#endif
// tiles between two additions of the waves' sums
#ifndef Q4K_STREAM_LDS_FLUSH
#define Q4K_STREAM_LDS_FLUSH 2
#endif
constexpr int kLdsFlush = Q4K_STREAM_LDS_FLUSH;
constexpr int kLdsWaves = 8;
constexpr int kLdsPieces = 16 * kBlockBytes / 16;   // 16-byte pieces of a wave's tile share: 144
constexpr int kLdsLoads = (kLdsPieces + 63) / 64;   // load instructions per wave and tile: 3

// The lane's 16-byte header at LDS byte address a and its two 16-byte code
// pieces at b and b + 64, complete on return.  One asm statement with its
// own wait: the compiler then sees no LDS read and adds no wait for the
// weight loads still in flight to the other ring slots.
__device__ __forceinline__ void lds_read_hdr_q2(uint32_t a, uint32_t b, uint4 &hdr, uint4 &q0, uint4 &q1) {
    u32x4_t x0, x1, x2;
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %4\n\t"
        "ds_read_b128 %2, %4 offset:64\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2)
        : "v"(a), "v"(b)
        : "memory");
    hdr = make_uint4(x0.x, x0.y, x0.z, x0.w);
    q0 = make_uint4(x1.x, x1.y, x1.z, x1.w);
    q1 = make_uint4(x2.x, x2.y, x2.z, x2.w);
}

template <int D, typename XT>
__global__ __launch_bounds__(64 * kLdsWaves, 1) void stream_lds_kernel(
    const uint8_t *__restrict__ w, const uint8_t *__restrict__ xc, float *__restrict__ y, int m, int64_t n, int64_t k,
    int64_t row_bytes, int64_t xc_bytes, const XT *__restrict__ x, int64_t flag_off) {
    constexpr int kSlot = kLdsLoads * 1024;
    __shared__ __align__(16) uint8_t wst[D][kLdsWaves][kSlot];
    __shared__ __align__(16) float4_t part[2][kLdsFlush][kLdsWaves][64];
    __shared__ int wflag[kLdsWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int nhalf = static_cast<int>(k / kStageK);
    // workgroup b: K part b % 2 of the tiles b / 2, b / 2 + gridDim.x / 2, ...
    const int kp = static_cast<int>(blockIdx.x & 1);
    const int tblk = static_cast<int>(blockIdx.x >> 1);
    const int tgrid = static_cast<int>(gridDim.x >> 1);
    const int hw0 = kp * (nhalf / 2) + 2 * wave;  // the wave's first half (even)
    const int sb = hw0 >> 1;                      // its super-block

    // the wave's two halves of activation fragments, sums and scales, in
    // registers (a lane whose token is past m reads zeros); the flags of
    // every half first
    const __amdgpu_buffer_rsrc_t ar = stream_rsrc(xc, static_cast<int>(xc_bytes));
    // (16 flag bytes per half: 128 dwords for 32 halves, one per thread)
    // (threads past them read past the descriptor's end: zeros, and no
    // branch, so that the wait for the flags comes after the loads below)
    const uint32_t flag_bits = __builtin_amdgcn_raw_buffer_load_b32(
        ar, static_cast<int>(threadIdx.x) < nhalf * 4 ? static_cast<int>(flag_off + 4 * threadIdx.x) : 0x40000000, 0, 0);
    const uint32_t a_off = col < m ? 0u : 0x40000000u;
    AStep as[2];
    PairSelect ps[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int soff = (hw0 + h) * kTileStageBytes;
#pragma unroll
        for (int f = 0; f < 8; ++f)
            as[h].f[f] = as_uint4(
                __builtin_amdgcn_raw_buffer_load_b128(ar, static_cast<int>(a_off + f * 1024 + lane * 16), soff, 0));
        as[h].sub = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(ar, kSubOff + col * 16, soff, 0));
        as[h].bias = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, kBiasOff + kq * 16, soff, 0));
        as[h].esc = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(ar, kEscOff + kq * 16, soff, 0));
        ps[h] = pair_select(2 * h + (kq >> 1));
    }
    const bool exact = workgroup_any(flag_bits, wflag, kLdsWaves);

    // the host keeps gridDim.x / 2 <= the number of tiles: every workgroup has one
    const int64_t ntiles = (n + 15) / 16;
    const int my_tiles = static_cast<int>((ntiles - 1 - tblk) / tgrid) + 1;
    auto tile_row0 = [&](int c) -> int64_t {
        return (static_cast<int64_t>(tblk) + static_cast<int64_t>(c) * tgrid) * 16;
    };
    if (exact) {
        // a flagged block: the workgroup's tiles (its K part) on the f32 path
        const int nsb = static_cast<int>(k / kBlockWeights);
        for (int c = 0; c < my_tiles; ++c) {
            const int64_t r0 = tile_row0(c);
            const int64_t r1 = r0 + 16 < n ? r0 + 16 : n;
            exact_tile<XT, float, true>(w, row_bytes, x, k, m, y, n, r0, r1, kp * nsb / 2, (kp + 1) * nsb / 2, wave,
                                        kLdsWaves);
        }
        return;
    }
    // the lane's descriptor offsets for the three loads of a tile: piece
    // p = 64 i + lane is row p / 9, bytes 16 (p % 9) of its super-block sb;
    // pieces past the 144th read past the descriptor's end (zeros)
    uint32_t voff[kLdsLoads];
#pragma unroll
    for (int i = 0; i < kLdsLoads; ++i) {
        const int p = 64 * i + lane;
        voff[i] = p < kLdsPieces ? static_cast<uint32_t>((p / 9) * row_bytes + sb * kBlockBytes + (p % 9) * 16)
                                 : 0x40000000u;
    }
    // tile c of this workgroup into ring slot b (a tile past the last: a
    // 0-byte descriptor, so the loads read zeros without a fetch)
    auto issue_stage = [&](int b, int c) {
        const bool live = c < my_tiles;
        const int64_t row0 = live ? tile_row0(c) : 0;
        const int64_t rows = n - row0 < 16 ? n - row0 : 16;
        const int nrec = __builtin_amdgcn_readfirstlane(live ? static_cast<int>(rows * row_bytes) : 0);
        const uint8_t *base =
            reinterpret_cast<const uint8_t *>(wave_uniform(reinterpret_cast<int64_t>(w + row0 * row_bytes)));
        const __amdgpu_buffer_rsrc_t r = stream_rsrc(base, nrec);
#pragma unroll
        for (int i = 0; i < kLdsLoads; ++i) buffer_load16_lds(r, &wst[b][wave][i * 1024], voff[i]);
    };
    const uint32_t rd_hdr = static_cast<uint32_t>(col * kBlockBytes);
    const uint32_t rd_q = rd_hdr + 16u + 16u * static_cast<uint32_t>(kq);

#pragma unroll
    for (int b = 0; b < D; ++b) issue_stage(b, b);
    // the activation loads (issued first) done, the weights still in flight;
    // without this the compiler waits for every load before the loop
    wait_vm<kLdsLoads * D>();
    for (int c = 0; c < my_tiles; c += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int cur = c + u;
            // tile cur's loads done (the D - 1 later tiles' stay in flight)
            wait_vm<kLdsLoads * (D - 1)>();
            const uint32_t slot = lds_addr(&wst[u][wave][0]);
            uint4 hdr, q[2];
            lds_read_hdr_q2(slot + rd_hdr, slot + rd_q, hdr, q[0], q[1]);
            issue_stage(u, cur + D);
            float4_t out = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                BOps bo;
                build_b_ops(bo, hdr, q[h], ps[h], kq);
                mfma_half(bo, as[h], out, kq);
            }
            const int d = cur % kLdsFlush;
            const int half = (cur / kLdsFlush) & 1;
            part[half][d][wave][lane] = out;
            if (d == kLdsFlush - 1 || cur + 1 == my_tiles) {
                lds_barrier();
                const int t = static_cast<int>(threadIdx.x);
                if (t < (d + 1) * 64) {
                    const int dd = t >> 6;
                    const int ln = t & 63;
                    float4_t sum = part[half][dd][0][ln];
#pragma unroll
                    for (int v = 1; v < kLdsWaves; ++v) sum += part[half][dd][v][ln];
                    const int64_t row = tile_row0(cur - d + dd) + (ln & 15);
                    if (row < n) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int tok = 4 * (ln >> 4) + r;
                            if (tok < m) unsafeAtomicAdd(y + static_cast<int64_t>(tok) * n + row, sum[r]);
                        }
                    }
                }
            }
            if (cur + 1 >= my_tiles) break;
        }
    }
    // the ring's last loads (past the last tile) land before the workgroup's
    // LDS is released
    wait_vm<0>();
}

__global__ __launch_bounds__(256) void f32_to_f16_kernel(const float *__restrict__ src, _Float16 *__restrict__ dst,
                                                          int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < count; i += stride) {
        dst[i] = static_cast<_Float16>(src[i]);
    }
}

// ------------------------------------------------------------- launchers
namespace {

// Super-blocks per stage (the workgroup has 2 waves per super-block).  More
// than 16 tokens at K <= 4096 take two (4 waves, one per SIMD): the kernel
// then has the whole register file of its SIMD, so 48-row workgroups keep 2-4
// token tiles without spilling to scratch (at four super-blocks, 8 waves of
// 256 registers, the 32- and 48-row shapes of 2-4 token tiles spill 48-64
// bytes per lane, and the spill stores reach HBM).  On the 9B gate two
// super-blocks alone took m = 32 from 24.6 to 22.2 us and m = 64 from 43.9 to
// 41.8 us, and the 48-row workgroups they allow m = 64 to 31.3 us; the 9B
// down (K = 12288) gained nothing from two.
#ifndef Q4K_BATCH_STAGE_SB
#define Q4K_BATCH_STAGE_SB 4
#endif
// super-blocks per stage for more than 16 tokens at K <= kBatchShortK
#ifndef Q4K_BATCH_STAGE_SB_SHORT
#define Q4K_BATCH_STAGE_SB_SHORT 2
#endif
// 1: long rows with one 16-row tile per CU halve K between two workgroups
// (dispatch_mt)
#ifndef Q4K_BATCH_HALVE_K
#define Q4K_BATCH_HALVE_K 1
#endif
// row tiles per workgroup at most for 2-4 token tiles with the short stage
#ifndef Q4K_BATCH_NT_SHORT
#define Q4K_BATCH_NT_SHORT 3
#endif
constexpr int64_t kBatchShortK = 4096;

// x: [m, k] of XT; y: [m, n] of YT.  An f16 output with K split across
// workgroups is accumulated in f32 in the call's scratch, then converted.
template <int NT, int MT, int S, typename XT, typename YT>
hipError_t launch_mfma_s(const uint8_t *w, const XT *x, YT *y, int m, int64_t n, int64_t k, int ksplit, Workspace &ws,
                         hipStream_t stream) {
    const int64_t nst = k / kStageK;
    const int64_t flag_off = nst * MT * kTileStageBytes;
    const int64_t bytes = flag_off + flag_bytes(nst, MT);
    constexpr bool kF32Out = std::is_same_v<YT, float>;
    const bool staged = !kF32Out && ksplit > 1;
    const int64_t ny = ksplit > 1 ? static_cast<int64_t>(m) * n : 0;
    const int64_t total = bytes + (staged ? ny * 4 : 0);
    if (ws.query) {
        if (total > ws.need) ws.need = total;
        return hipSuccess;
    }
    uint8_t *xc = nullptr;
    bool owned = false;
    hipError_t e = ws_acquire(ws, total, stream, &xc, &owned);
    if (e != hipSuccess) return e;
    float *acc_y = nullptr;  // where the matrix-core kernel accumulates with atomics
    if constexpr (kF32Out) acc_y = y;
    if (staged) acc_y = reinterpret_cast<float *>(xc + bytes);
    const int64_t prep_threads = nst * 16 * MT * 32;
    const int64_t prep_blocks = (prep_threads + 255) / 256;
    hipLaunchKernelGGL(x_prep_kernel<XT>, dim3(static_cast<unsigned>(prep_blocks)), dim3(256), 0, stream, x, xc,
                       xc + flag_off, reinterpret_cast<uint32_t *>(acc_y), m, MT, k, ny);
    e = hipGetLastError();
    if (e == hipSuccess) {
        const int64_t nrb = (n + 16 * NT - 1) / (16 * NT);
        const dim3 grid(static_cast<unsigned>(nrb * ksplit));
        const int64_t rb = (k / kBlockWeights) * kBlockBytes;
        if (staged) {
            hipLaunchKernelGGL((batched_mfma_kernel<NT, MT, S, float, XT>), grid, dim3(128 * S), 0, stream, w, xc,
                               acc_y, m, n, k, rb, ksplit, bytes, x, flag_off);
            e = hipGetLastError();
            if (e == hipSuccess) {
                const int64_t need = (ny + 255) / 256;
                hipLaunchKernelGGL(f32_to_f16_kernel, dim3(static_cast<unsigned>(need < 4096 ? need : 4096)),
                                   dim3(256), 0, stream, acc_y, reinterpret_cast<_Float16 *>(y), ny);
                e = hipGetLastError();
            }
        } else {
            hipLaunchKernelGGL((batched_mfma_kernel<NT, MT, S, YT, XT>), grid, dim3(128 * S), 0, stream, w, xc, y, m,
                               n, k, rb, ksplit, bytes, x, flag_off);
            e = hipGetLastError();
        }
    }
    const hipError_t f = ws_release(xc, owned, stream);
    return e != hipSuccess ? e : f;
}

// tiles in flight per wave (ring slots + 1) of the weight-streaming kernel
// when two workgroups split K, and whether they do (launch_stream)
#ifndef Q4K_STREAM_KP_NB
#define Q4K_STREAM_KP_NB 2
#endif
#ifndef Q4K_STREAM_KPARTS
#define Q4K_STREAM_KPARTS 1
#endif
#ifndef Q4K_STREAM_NB
#define Q4K_STREAM_NB 2
#endif

// m <= 16 tokens, k <= kStreamMaxK: the activation operands prepared once,
// then the weight-streaming kernel (no split of K, no atomics).
template <typename XT, typename YT>
hipError_t launch_stream(const uint8_t *w, const XT *x, YT *y, int m, int64_t n, int64_t k, Workspace &ws,
                         hipStream_t stream) {
    const int64_t nhalf = k / kStageK;
    const int64_t flag_off = nhalf * kTileStageBytes;
    const int64_t bytes = flag_off + flag_bytes(nhalf, 1);
    if (ws.query) {
        if (bytes > ws.need) ws.need = bytes;
        return hipSuccess;
    }
    uint8_t *xc = nullptr;
    bool owned = false;
    hipError_t e = ws_acquire(ws, bytes, stream, &xc, &owned);
    if (e != hipSuccess) return e;
    const int64_t ntiles = (n + 15) / 16;
    const int64_t cus = device_cu_count();
    // Few tiles per CU at K = 4096 (the 9B gate: 3): each workgroup's
    // activation fragments (256 KB at 16 tokens) weigh as much as its
    // weights, so two workgroups split K instead, each loading half of them
    // for twice as many tiles; their partial tiles are added into y (zeroed
    // by the preparation kernel), two addends per output, whose sum does not
    // depend on their order.
    const bool kparts = std::is_same_v<YT, float> && Q4K_STREAM_KPARTS && nhalf == kStreamMaxHalves &&
                        ntiles <= 8 * cus && cus % 2 == 0;
    const int64_t prep_blocks = (nhalf * 16 * 32 + 255) / 256;
    hipLaunchKernelGGL(x_prep_kernel<XT>, dim3(static_cast<unsigned>(prep_blocks)), dim3(256), 0, stream, x, xc,
                       xc + flag_off, kparts ? reinterpret_cast<uint32_t *>(y) : static_cast<uint32_t *>(nullptr), m,
                       1, k, kparts ? static_cast<int64_t>(m) * n : int64_t{0});
    e = hipGetLastError();
    if (e == hipSuccess && kparts) {
        // two halves per wave, eight waves per K part, one workgroup per CU
        const int64_t tiles2 = 2 * ntiles;
        const dim3 grid(static_cast<unsigned>(tiles2 < cus ? tiles2 : cus));
        const int64_t rb = (k / kBlockWeights) * kBlockBytes;
        if constexpr (std::is_same_v<YT, float>) {
            if (Q4K_STREAM_LDS) {
                hipLaunchKernelGGL((stream_lds_kernel<Q4K_STREAM_LDS_D, XT>), grid, dim3(64 * kLdsWaves), 0, stream, w,
                                   xc, y, m, n, k, rb, bytes, x, flag_off);
            } else {
                hipLaunchKernelGGL((stream_mfma_kernel<2, Q4K_STREAM_KP_NB, float, XT, 2>), grid, dim3(64 * 8), 0, stream,
                                   w, xc, y, m, n, k, rb, bytes, x, flag_off);
            }
        }
        e = hipGetLastError();
    } else if (e == hipSuccess) {
        // halves per wave: one up to 16 halves (K = 2048), then four (eight
        // waves of 256 registers); two spill at the 128 registers of 16 waves
        const int H = nhalf <= kStreamMaxWaves ? 1 : 4;
        const int nw = static_cast<int>((nhalf + H - 1) / H);
        const int64_t cap = cus * (H == 1 && nw <= 8 ? 2 : 1);
        const dim3 grid(static_cast<unsigned>(ntiles < cap ? ntiles : cap));
        const int64_t rb = (k / kBlockWeights) * kBlockBytes;
        constexpr int NB = Q4K_STREAM_NB;
        if (H == 1) {
            hipLaunchKernelGGL((stream_mfma_kernel<1, NB, YT, XT>), grid, dim3(64 * nw), 0, stream, w, xc, y, m, n, k,
                               rb, bytes, x, flag_off);
        } else {
            hipLaunchKernelGGL((stream_mfma_kernel<4, NB, YT, XT>), grid, dim3(64 * nw), 0, stream, w, xc, y, m, n, k,
                               rb, bytes, x, flag_off);
        }
        e = hipGetLastError();
    }
    const hipError_t f = ws_release(xc, owned, stream);
    return e != hipSuccess ? e : f;
}

// Rows per workgroup (16*NT) and the split of K across workgroups.  Each
// workgroup reads its whole K range of activations (16*MT tokens x 4 bytes
// per activation) besides its weights (0.5625 bytes per weight), so when
// there are too few rows for every CU to get several, rows are grouped into
// larger blocks and K is split across workgroups instead (their partial tiles
// are then added into y with atomics).  With four super-blocks per stage (8
// waves of 256 registers) the register budget caps the rows per workgroup at
// 64 / 48 / 32 / 32 for 1 / 2 / 3 / 4 token tiles (the 48-row shape of 2
// tiles and the 32-row shape of 4 spill a few registers and are still the
// faster ones: each row block re-reads fewer activations); with two (4 waves
// of 512 registers, more than 16 tokens at K <= 4096) 48 rows fit 2-4 token
// tiles, and a 12,288-row matrix is then one row block per CU instead of 1.5.
#ifndef Q4K_BATCH_NT_CAP
#define Q4K_BATCH_NT_CAP 4
#endif
template <int MT, int S, int kNtMax, typename XT, typename YT>
hipError_t dispatch_rows(const uint8_t *w, const XT *x, YT *y, int m, int64_t n, int64_t k, Workspace &ws,
                         hipStream_t stream) {
    const int64_t cus = device_cu_count();
    const int64_t nsb = k / kBlockWeights;
    const int64_t per = n / (16 * cus);  // row tiles per CU with one row block each
    if (per >= 1 || nsb < 2) {
        const int64_t nt = per < 1 ? 1 : (per > kNtMax ? kNtMax : per);
        if (nt >= 4) return launch_mfma_s<kNtMax, MT, S, XT, YT>(w, x, y, m, n, k, 1, ws, stream);
        if (nt == 3) return launch_mfma_s<(kNtMax < 3 ? kNtMax : 3), MT, S, XT, YT>(w, x, y, m, n, k, 1, ws, stream);
        if (nt == 2) return launch_mfma_s<(kNtMax < 2 ? kNtMax : 2), MT, S, XT, YT>(w, x, y, m, n, k, 1, ws, stream);
        return launch_mfma_s<1, MT, S, XT, YT>(w, x, y, m, n, k, 1, ws, stream);
    }
    // fewer than 16 rows per CU: the largest row blocks, K split to fill the CUs
    const int64_t nrb = (n + 16 * kNtMax - 1) / (16 * kNtMax);
    int64_t ksplit = (cus + nrb - 1) / nrb;
    if (ksplit > nsb) ksplit = nsb;
    return launch_mfma_s<kNtMax, MT, S, XT, YT>(w, x, y, m, n, k, static_cast<int>(ksplit), ws, stream);
}

template <int MT, typename XT, typename YT>
hipError_t dispatch_mt(const uint8_t *w, const XT *x, YT *y, int m, int64_t n, int64_t k, Workspace &ws,
                       hipStream_t stream) {
    constexpr int kNtMax0 = MT == 1 ? 4 : (MT == 2 ? 3 : 2);
    constexpr int kNtMax = kNtMax0 < Q4K_BATCH_NT_CAP ? kNtMax0 : Q4K_BATCH_NT_CAP;
    constexpr int kNtShort0 = MT == 1 ? kNtMax0 : Q4K_BATCH_NT_SHORT;
    constexpr int kNtShort = kNtShort0 < Q4K_BATCH_NT_CAP ? kNtShort0 : Q4K_BATCH_NT_CAP;
    const int64_t cus = device_cu_count();
    // Long rows with exactly one 16-row tile per CU (the 9B down: 4096 rows,
    // K = 12288): every workgroup would read its whole K range of
    // activations for 16 rows.  32-row workgroups with K halved between two
    // of them read half as much per row for the same number of workgroups;
    // the two partial tiles are added into y (zeroed first) with f32 atomics,
    // and with exactly two addends (0 + a, then + b, or the other way round)
    // the sum is the same whatever their order, so the result stays
    // reproducible.
    const bool halve_k = Q4K_BATCH_HALVE_K && k > kBatchShortK && n / (16 * cus) == 1 &&
                         2 * ((n + 31) / 32) <= cus && k / kBlockWeights >= 2;
    if constexpr (MT == 1) {
        // a row tile for every CU: the weight-streaming kernel
        if (k <= kStreamMaxK && (n + 15) / 16 >= cus) return launch_stream(w, x, y, m, n, k, ws, stream);
        if (halve_k) return launch_mfma_s<2, MT, Q4K_BATCH_STAGE_SB, XT, YT>(w, x, y, m, n, k, 2, ws, stream);
        return dispatch_rows<MT, Q4K_BATCH_STAGE_SB, kNtMax>(w, x, y, m, n, k, ws, stream);
    } else {
        if (k <= kBatchShortK) {
            return dispatch_rows<MT, Q4K_BATCH_STAGE_SB_SHORT, kNtShort>(w, x, y, m, n, k, ws, stream);
        }
        if (halve_k) return launch_mfma_s<2, MT, Q4K_BATCH_STAGE_SB_SHORT, XT, YT>(w, x, y, m, n, k, 2, ws, stream);
        return dispatch_rows<MT, Q4K_BATCH_STAGE_SB, kNtMax>(w, x, y, m, n, k, ws, stream);
    }
}

}  // namespace

template <typename XT, typename YT>
hipError_t batched_slices(const uint8_t *w, const XT *x, YT *y, int64_t m, int64_t n, int64_t k, Workspace &ws,
                          hipStream_t stream) {
    hipError_t e = hipSuccess;
    // up to 64 tokens per launch; the weights are re-read per 64-token slice
    for (int64_t t0 = 0; t0 < m; t0 += 64) {
        const int mt = static_cast<int>(m - t0 < 64 ? m - t0 : 64);
        const XT *xs = x + t0 * k;
        YT *ys = y + t0 * n;
        if (mt <= 16) e = dispatch_mt<1>(w, xs, ys, mt, n, k, ws, stream);
        else if (mt <= 32) e = dispatch_mt<2>(w, xs, ys, mt, n, k, ws, stream);
        else if (mt <= 48) e = dispatch_mt<3>(w, xs, ys, mt, n, k, ws, stream);
        else e = dispatch_mt<4>(w, xs, ys, mt, n, k, ws, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv_batched_dt(const uint8_t *w, const void *x, bool x_f16, void *y, bool y_f16, int64_t m,
                                  int64_t n, int64_t k, Workspace &ws, hipStream_t stream) {
    if (m == 0 || n == 0) return hipSuccess;
    if (ws.query && (k == 0 || m == 1)) return hipSuccess;  // no scratch on these paths
    if (k == 0) {
        return y_f16 ? launch_fill_zero_f16(static_cast<_Float16 *>(y), m * n, stream)
                     : launch_fill_zero(static_cast<float *>(y), m * n, stream);
    }
    if (m == 1) return launch_gemv_dt(w, x, x_f16, y, y_f16, n, k, stream);
    // A few tokens: the streaming GEMV with the codes decoded once per token
    // pair, no scratch.  Three or four tokens over many rows (four 16-row
    // tiles per CU or more) go to the weight-streaming matrix-core kernel
    // instead: there the decode work of a second token pair outweighs its
    // activation preparation.
    const bool few = (m <= kTokensMax && k <= kTokensMaxK) || (m == 2 && k <= kTokensSplitMaxK);
    const bool many_rows = m > 2 && k <= kStreamMaxK && (n + 15) / 16 >= 4 * static_cast<int64_t>(device_cu_count());
    if (few && !many_rows) {
        if (ws.query) return hipSuccess;
        return launch_gemv_tokens(w, x, x_f16, y, y_f16, m, n, k, stream);
    }
    // Prefill sizes with f16 activations: the prefill GEMM (exact f16
    // operands, 128-token tiles) is the faster kernel there.  It reads x in
    // 16-byte pieces, so it takes only a 16-byte aligned x; a size query,
    // which does not know x, makes room for either path.
    if (x_f16 && m >= kPrefillMinTokens && k <= kPrefillMaxK) {
        if (ws.query) {
            const hipError_t e = launch_prefill(w, static_cast<const _Float16 *>(x), y, y_f16, m, n, k, ws, stream);
            if (e != hipSuccess) return e;
        } else if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
            return launch_prefill(w, static_cast<const _Float16 *>(x), y, y_f16, m, n, k, ws, stream);
        }
    }
    using H = _Float16;
    if (x_f16 && y_f16) return batched_slices(w, static_cast<const H *>(x), static_cast<H *>(y), m, n, k, ws, stream);
    if (x_f16) return batched_slices(w, static_cast<const H *>(x), static_cast<float *>(y), m, n, k, ws, stream);
    if (y_f16) return batched_slices(w, static_cast<const float *>(x), static_cast<H *>(y), m, n, k, ws, stream);
    return batched_slices(w, static_cast<const float *>(x), static_cast<float *>(y), m, n, k, ws, stream);
}

hipError_t launch_gemv_batched(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                               hipStream_t stream) {
    Workspace ws;
    return launch_gemv_batched_dt(w, x, false, y, false, m, n, k, ws, stream);
}

}  // namespace q4k
