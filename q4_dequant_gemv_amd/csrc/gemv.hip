// Batch-1 Q4_K GEMV and the fused gate/up SwiGLU GEMV.
//
// The operation is the fused dequant+GEMV over raw Q4K bytes of "Struct
// WgslForwardPass" (upload_q4k_weight) and the try_q4k_soa_gemv /
// try_q4k_soa_fused_swiglu entry points of the qualia_core_db cuda_lane
// module, at M == 1 (the decode phase of resolveMatmulPhase in
// "@simulatte/doppler 0.1.7 -> 0.1.8", matmul-selection.js).
//
// Design for gfx950.  At batch 1 every weight byte is used once, so the
// kernel is an HBM stream: each lane owns one 64-weight group (the code bytes
// of a sub-block pair, 32 contiguous bytes) of a row, plus the super-block's
// 16-byte header, and a row of K weights is covered by LPR = K/64 lanes (16,
// 32 or 64 at K = 1024, 2048, 4096).  Rows are handed to waves round-robin by
// a persistent grid sized to the resident capacity.  Wider rows (K = 8192 to
// 16384) are split over S = K/4096 waves of one workgroup, each holding its
// slice of the activations in registers; their partial row sums meet in LDS.
//
// Arithmetic per weight has to stay near one vector instruction, so the dot
// product is done in integers: each 64-activation group is converted once per
// workgroup to X = rint(x * 2^(21-e)) (e = exponent of the group's largest
// magnitude, |X| <= 2^22) and split into three signed bytes.  The codes are
// 0..15, so v_dot4_i32_i8 multiplies four codes by four activation bytes and
// accumulates exactly; per 8 weights that is 3 unpack + 6 dot instructions.
// Per sub-block s the exact integer S_s = sum q X combines the three limbs
// (|S_s| < 2^31 by construction), and the sub-block contributes
//     scale * (d*sc_s * S_s - dmin*m_s * sum_{e in s} X_e)
// in f32.  The min term uses the same integers X as the code term, so a
// sub-block whose weights are all zero still contributes zero.  Each x is
// represented to within 2^-22 of its group's largest magnitude, and the f32
// roundings are a few 2^-24 of the terms, so the error stays far inside the
// 2e-4 * sum|w x| bound unless, within one 64-activation group, the largest
// |x| exceeds the |w|-weighted typical |x| by several hundred times.
//
// Row partial sums are reduced across the LPR lanes of the row with DPP and
// permlane swaps (no LDS); the workgroup's activations are converted once into
// LDS and then held in registers for the whole row stream.
//
// The same kernels serve a batched call of a few tokens: each wave holds two
// tokens' activation registers and decodes every weight group once for both,
// and waves of one workgroup that take the same rows for different token
// pairs share the row's bytes through the caches.
#include <float.h>
#include <math.h>

#include <atomic>
#include <type_traits>

#include "launch.h"
#include "q4k_device.h"
#include "q4k_int_dot.h"

namespace q4k {

// A weight format of the streaming kernels: what one lane loads for its
// 64-weight group of a row, where those bytes sit, and their dot product with
// the group's activations.  Lanes past the row's last group (K/64 not a power
// of two) read group 0 again and drop it.
//
// Q4_K: the group is sub-block pair (2g, 2g+1) of a 144-byte super-block; the
// lane loads the super-block's 16-byte header and the group's 32 code bytes.
struct Q4KFormat {
    // Single-token kernels stage the weight stream through LDS: a wave's
    // iteration (whole rows, contiguous bytes) arrives by 16-byte loads that
    // each cover a contiguous kilobyte, and each lane then reads its header
    // and code chunks from LDS (fetch).
    static constexpr bool kStaged = true;
    static constexpr int kGroupBytes = 36;  // 144 bytes per 4 groups of 64 weights
    struct Lane {
        uint32_t off_hdr;  // byte offset of the super-block header
        uint32_t off_qa;   // byte offset of the group's first 16 code bytes
        PairSelect ps;
        int j;             // group index (clamped)
        bool ok;           // the group exists
    };
    struct Loads {
        uint4 hdr, qa, qb;
    };
    static int64_t row_bytes(int64_t k) { return (k / kBlockWeights) * kBlockBytes; }
    static __device__ __forceinline__ Lane lane(int j, int ngroups, uint32_t row_off) {
        Lane g;
        g.ok = j < ngroups;
        g.j = g.ok ? j : 0;
        g.ps = pair_select(g.j & 3);
        g.off_hdr = row_off + static_cast<uint32_t>(g.j >> 2) * kBlockBytes;
        g.off_qa = g.off_hdr + 16u + 32u * static_cast<uint32_t>(g.j & 3);
        return g;
    }
    static __device__ __forceinline__ void issue(Loads &l, __amdgpu_buffer_rsrc_t r, const Lane &g) {
        l.hdr = buffer_load16(r, g.off_hdr);
        l.qa = buffer_load16(r, g.off_qa);
        l.qb = buffer_load16(r, g.off_qa + 16u);
    }
    // the same bytes from a staged copy of the iteration at LDS byte address
    // `stage` (headers and code chunks sit at multiples of 16 bytes)
    static __device__ __forceinline__ void fetch(Loads &l, uint32_t stage, const Lane &g) {
        lds_read_3x16(stage + g.off_hdr, stage + g.off_qa, l.hdr, l.qa, l.qb);
    }
    // sum over the group of w * x in units of the group's activation scale
    static __device__ __forceinline__ float dot(const Loads &l, const Lane &g, const XRegs &xr) {
        GroupCodes c;
        decode_group(l.hdr, l.qa, l.qb, g.ps, c);
        return group_dot(c, xr);
    }
    // the same for MT tokens, the codes decoded once; acc[t] in units of 1
    template <int MT>
    static __device__ __forceinline__ void dot_tokens(const Loads &l, const Lane &g, const XRegs (&xr)[MT], bool active,
                                                      float (&acc)[MT]) {
        GroupCodes c;
        decode_group(l.hdr, l.qa, l.qb, g.ps, c);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            acc[t] = 0.0f;
            if (active) acc[t] = xr[t].scale * group_dot(c, xr[t]);
        }
    }
    // sum over the group of w * x in f32, each weight on its own (the f32
    // path); xs: the group's 64 activations (registers or memory)
    // (after: see exact_group_dot)
    template <typename T>
    static __device__ __forceinline__ float dot_exact(const Loads &l, const Lane &g, const T *xs, float after) {
        GroupCodes c;
        decode_group(l.hdr, l.qa, l.qb, g.ps, c);
        return exact_group_dot(c, xs, after);
    }
    template <int MT, typename T>
    static __device__ __forceinline__ void dot_tokens_exact(const Loads &l, const Lane &g, const T *const (&xs)[MT],
                                                            bool active, float after, float (&acc)[MT]) {
        GroupCodes c;
        decode_group(l.hdr, l.qa, l.qb, g.ps, c);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            acc[t] = 0.0f;
            if (active) acc[t] = exact_group_dot(c, xs[t], t == 0 ? after : acc[t - 1]);
        }
    }
};

// Q8_0: 34-byte blocks of 32 weights, an f16 scale d then 32 signed bytes q,
// w = d * q.  The lane's 64-weight group is two blocks, 68 bytes starting at
// 68*j, dword-aligned whenever the row is (K % 64 == 0 and a 4-byte aligned
// matrix): 17 dwords, loaded as four 16-byte loads and one 4-byte load.  The
// second block's codes are dword-aligned; the first block's start two bytes
// into a dword and are realigned with v_alignbyte.  The codes are signed
// bytes, so v_dot4_i32_i8 multiplies them with the activation limbs directly.
// A limb sum stays within 32 * 128 * 128 = 2^19, but the recombined sum of a
// block reaches 2^34, beyond int32: the three limb sums are converted to f32
// (exactly) and combined with two FMAs, one rounding each (a relative 2^-24
// of the block's sum).
struct Q8_0Format {
    // groups start at multiples of 68 bytes, not of 16: no LDS staging
    static constexpr bool kStaged = false;
    static constexpr int kGroupBytes = 68;
    static constexpr int kBlockWeights = 32;
    static constexpr int kBlockBytes = 34;
    struct Lane {
        uint32_t off;  // byte offset of the group's first block
        int j;
        bool ok;
    };
    struct Loads {
        uint4 a, b, c, d;
        uint32_t e;
    };
    static int64_t row_bytes(int64_t k) { return (k / kBlockWeights) * kBlockBytes; }
    static __device__ __forceinline__ Lane lane(int j, int ngroups, uint32_t row_off) {
        Lane g;
        g.ok = j < ngroups;
        g.j = g.ok ? j : 0;
        g.off = row_off + 68u * static_cast<uint32_t>(g.j);
        return g;
    }
    static __device__ __forceinline__ void issue(Loads &l, __amdgpu_buffer_rsrc_t r, const Lane &g) {
        l.a = buffer_load16(r, g.off);
        l.b = buffer_load16(r, g.off + 16u);
        l.c = buffer_load16(r, g.off + 32u);
        l.d = buffer_load16(r, g.off + 48u);
        l.e = buffer_load4(r, g.off + 64u);
    }
    static __device__ __forceinline__ float dot(const Loads &l, const Lane &, const XRegs &xr) {
        const uint32_t dw[17] = {l.a.x, l.a.y, l.a.z, l.a.w, l.b.x, l.b.y, l.b.z, l.b.w, l.c.x,
                                 l.c.y, l.c.z, l.c.w, l.d.x, l.d.y, l.d.z, l.d.w, l.e};
        const float d0 = half_bits_to_float(dw[0]);
        const float d1 = half_bits_to_float(dw[8] >> 16);
        int a00 = 0, a01 = 0, a02 = 0, a10 = 0, a11 = 0, a12 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // bytes 2+4i .. 5+4i of the group: codes 4i .. 4i+3 of the first block
            const int q0 = static_cast<int>(__builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2));
            const int q1 = static_cast<int>(dw[9 + i]);
            a00 = __builtin_amdgcn_sdot4(q0, static_cast<int>(xr.limb[0][0][i]), a00, false);
            a01 = __builtin_amdgcn_sdot4(q0, static_cast<int>(xr.limb[0][1][i]), a01, false);
            a02 = __builtin_amdgcn_sdot4(q0, static_cast<int>(xr.limb[0][2][i]), a02, false);
            a10 = __builtin_amdgcn_sdot4(q1, static_cast<int>(xr.limb[1][0][i]), a10, false);
            a11 = __builtin_amdgcn_sdot4(q1, static_cast<int>(xr.limb[1][1][i]), a11, false);
            a12 = __builtin_amdgcn_sdot4(q1, static_cast<int>(xr.limb[1][2][i]), a12, false);
        }
        const float s0 = fmaf(static_cast<float>(a02), 65536.0f, fmaf(static_cast<float>(a01), 256.0f,
                                                                        static_cast<float>(a00)));
        const float s1 = fmaf(static_cast<float>(a12), 65536.0f, fmaf(static_cast<float>(a11), 256.0f,
                                                                        static_cast<float>(a10)));
        return d0 * s0 + d1 * s1;
    }
    // the f32 path: w = d * q (exact in f32) times x, each product rounded once
    template <typename T>
    static __device__ __forceinline__ float dot_exact(const Loads &l, const Lane &, const T *xs, float after) {
        const uint32_t dw[17] = {l.a.x, l.a.y, l.a.z, l.a.w, l.b.x, l.b.y, l.b.z, l.b.w, l.c.x,
                                 l.c.y, l.c.z, l.c.w, l.d.x, l.d.y, l.d.z, l.d.w, l.e};
        const float d0 = half_bits_to_float(dw[0]);
        const float d1 = half_bits_to_float(dw[8] >> 16);
        float a0 = 0.0f, a1 = 0.0f, nf = 0.0f;
        // a quarter of the activations at a time, each quarter summed on its
        // own, and NaN for a non-finite activation, as exact_group_dot
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const global_ptr<T> p = opaque_after(xs, h == 0 ? after : a0, a1);
            float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
            for (int i = 2 * h; i < 2 * h + 2; ++i) {
                const uint32_t q0 = __builtin_amdgcn_alignbyte(dw[i + 1], dw[i], 2);
                const uint32_t q1 = dw[9 + i];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float w0 = d0 * static_cast<float>(static_cast<int8_t>((q0 >> (8 * b)) & 0xffu));
                    const float w1 = d1 * static_cast<float>(static_cast<int8_t>((q1 >> (8 * b)) & 0xffu));
                    const float x0 = static_cast<float>(p[4 * i + b]);
                    const float x1 = static_cast<float>(p[32 + 4 * i + b]);
                    s0 = fmaf(w0, x0, s0);
                    s1 = fmaf(w1, x1, s1);
                    nf = fmaf(x0, 0.0f, fmaf(x1, 0.0f, nf));
                }
            }
            a0 += s0;
            a1 += s1;
        }
        return (a0 + a1) + nf;
    }
};

// Q8_0 staged through LDS like Q4_K: a wave's iteration (whole rows,
// contiguous bytes) arrives by direct-to-LDS loads, then each lane reads its
// group's 17 dwords from LDS (dword-aligned: lane stride 68 bytes, 17 dwords,
// an odd count, so the 64 lanes' reads fall in distinct banks).  Used where
// every iteration starts on a 16-byte boundary: rows of a multiple of 256
// weights (68 * K / 64 bytes, a multiple of 16) in a 16-byte aligned matrix,
// at most 4096 weights long, or 8193-12288 weights (the three-slice split
// kernel; the other split shapes would need more LDS than a CU has for their
// rings of 4352-byte slices).
#ifndef Q4K_Q8_0_STAGE
#define Q4K_Q8_0_STAGE 1
#endif
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
struct Q8_0StagedFormat : Q8_0Format {
    static constexpr bool kStaged = true;
    static __device__ __forceinline__ void fetch(Loads &l, uint32_t stage, const Lane &g) {
        const uint32_t a = stage + g.off;
        u32x2_t p0, p1, p2, p3, p4, p5, p6, p7;
        uint32_t e;
        // one asm statement with its own wait: the compiler sees no LDS read
        // and adds no wait for the loads still in flight to other slots
        asm volatile(
            "ds_read2_b32 %0, %9 offset1:1\n\t"
            "ds_read2_b32 %1, %9 offset0:2 offset1:3\n\t"
            "ds_read2_b32 %2, %9 offset0:4 offset1:5\n\t"
            "ds_read2_b32 %3, %9 offset0:6 offset1:7\n\t"
            "ds_read2_b32 %4, %9 offset0:8 offset1:9\n\t"
            "ds_read2_b32 %5, %9 offset0:10 offset1:11\n\t"
            "ds_read2_b32 %6, %9 offset0:12 offset1:13\n\t"
            "ds_read2_b32 %7, %9 offset0:14 offset1:15\n\t"
            "ds_read_b32 %8, %9 offset:64\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(p0), "=&v"(p1), "=&v"(p2), "=&v"(p3), "=&v"(p4), "=&v"(p5), "=&v"(p6), "=&v"(p7), "=&v"(e)
            : "v"(a)
            : "memory");
        l.a = make_uint4(p0.x, p0.y, p1.x, p1.y);
        l.b = make_uint4(p2.x, p2.y, p3.x, p3.y);
        l.c = make_uint4(p4.x, p4.y, p5.x, p5.y);
        l.d = make_uint4(p6.x, p6.y, p7.x, p7.y);
        l.e = e;
    }
};

// One row's weight bytes for one lane, per matrix.
template <class F, int NMAT>
struct RowLoads {
    typename F::Loads m[NMAT];
};

// Issues one row's loads from descriptors based at `base` (wave-uniform) that
// cover `nrec` bytes: loads at or past nrec return zeros, so a row past the
// end costs no memory traffic and needs no branch.
template <class F, int NMAT>
__device__ __forceinline__ void issue_row(RowLoads<F, NMAT> &b, const uint8_t *w, const uint8_t *wu, int64_t base,
                                          int nrec, const typename F::Lane &g) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) F::issue(b.m[mt], stream_rsrc((mt == 0 ? w : wu) + base, nrec), g);
}

// The lane's share of the row, per matrix: sum over its group of w * x.
template <class F, int NMAT>
__device__ __forceinline__ void lane_dot(const RowLoads<F, NMAT> &b, const typename F::Lane &g, const XRegs &xr,
                                         bool active, float (&acc)[NMAT]) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
        acc[mt] = 0.0f;
        if (active) acc[mt] = xr.scale * F::dot(b.m[mt], g, xr);
    }
}

// The same on the f32 path: xs is the lane's group of the activations.
// after: see exact_group_dot.
template <class F, int NMAT, typename T>
__device__ __forceinline__ void lane_dot_exact(const RowLoads<F, NMAT> &b, const typename F::Lane &g, const T *xs,
                                               bool active, float after, float (&acc)[NMAT]) {
#pragma unroll
    for (int mt = 0; mt < NMAT; ++mt) {
        acc[mt] = 0.0f;
        if (active) acc[mt] = F::dot_exact(b.m[mt], g, xs, mt == 0 ? after : acc[mt - 1]);
    }
}

// ---------------------------------------------------------------- K <= 4096
// LPR lanes per row (power of two, <= 64; LPR >= K/64), 64/LPR rows per wave
// iteration.  SWIGLU reads a second matrix `wu` of the same shape and writes
// silu(W x) * (Wu x).  Each wave rotates NB register buffers: while one row is
// decoded, multiplied and reduced, the next NB-1 rows' loads are in flight;
// the first rows are issued before the activations are prepared.  Wave
// iterations are dealt round-robin over the persistent grid.
// Up to kMaxMats matrices of the same k against one x in a single launch (the
// q, k and v projections of a decode step, say).  Matrix i owns the wave
// iterations [it_begin[i], it_begin[i+1]); its last iteration covers
// tail_bytes of weights.  r[i], if set, is added to each output (a residual).
// 1: single-token Q4_K streams read their weights through LDS (see
// gemv_kernel); 0: straight into registers, as the other streams do.
#ifndef Q4K_STAGE
#define Q4K_STAGE 1
#endif

constexpr int kMaxMats = 8;
struct MatTable {
    const uint8_t *w[kMaxMats];
    void *y[kMaxMats];  // YT [n] each
    const float *r[kMaxMats];
    int64_t n[kMaxMats];
    void *y_gate[kMaxMats];  // with head_log2: the gate half of each head's rows
    int head_log2[kMaxMats];
    int it_begin[kMaxMats + 1];
    int tail_bytes[kMaxMats];
    int count;
};

// XT, YT: activation and output element types (float or _Float16).  RES:
// some matrix of the table has a residual.  Only then does the store path
// load it: a load there, though rarely executed, makes the compiler's wait
// counts in the streaming loop more conservative.  RPG: rows per lane group
// and iteration (the lane takes its group of RPG rows, 64/LPR rows apart),
// which puts RPG rows per buffer in flight with the same activation
// registers.  QG: some matrix of the table de-interleaves its output per
// head (y_gate set); only then does the store path remap rows.
//
// MT, TP: several tokens (a small batch, x [ntok][K], y [ntok][n], one
// matrix).  A wave holds the activation registers of MT tokens and decodes
// each weight group once for all of them; TP waves of a workgroup (adjacent
// wave indices) take the same wave iteration for token tiles 0 .. TP-1, so a
// row's bytes come from HBM once and reach the other waves from the caches.
// Tokens past ntok in the last tile repeat token ntok-1 and are not stored.
template <class F, typename XT, typename YT, int LPR, bool SWIGLU, bool RES, int NB, int BLOCK, int MIN_WAVES,
          int RPG, bool QG = false, int MT = 1, int TP = 1>
__global__ __launch_bounds__(BLOCK, MIN_WAVES) void gemv_kernel(const MatTable mt, const uint8_t *__restrict__ wu,
                                                                const XT *x, int ngroups, int64_t row_bytes,
                                                                int ntok) {
    static_assert(NB >= 2, "at least one row in flight");
    static_assert(MT * TP == 1 || (!SWIGLU && !RES && !QG && RPG == 1), "token tiles: plain single-matrix GEMV");
    constexpr int NMAT = SWIGLU ? 2 : 1;
    constexpr int kRowsPerGroup = kWave / LPR;  // rows per wave and row slot q
    constexpr int kRowsPerWave = RPG * kRowsPerGroup;
    constexpr int kWavesPerBlock = BLOCK / kWave;
    static_assert(kWavesPerBlock % TP == 0, "whole token-tile groups per workgroup");
    constexpr int kIterWaves = kWavesPerBlock / TP;  // waves of a workgroup with distinct iterations
    constexpr int kTok = MT * TP;
    extern __shared__ __align__(16) unsigned char smem[];
    XGroup *xg = reinterpret_cast<XGroup *>(smem);
    // Single-token Q4_K streams stage the weights through LDS: a ring of
    // kSlots = NB - 1 slots per wave (one per matrix each) holds the wave's
    // next iterations (kIterBytes at most: RPG * 64 groups).
    constexpr bool kStage = F::kStaged && kTok == 1 && Q4K_STAGE != 0;
    constexpr int kSlots = kStage ? NB - 1 : 1;
    constexpr int kIterBytes = RPG * kWave * F::kGroupBytes;
    constexpr int kDma = stage_loads<kIterBytes>();
    __shared__ __align__(16)
        uint8_t stage[kSlots][kStage ? NMAT : 1][kStage ? kWavesPerBlock : 1][kStage ? kIterBytes : 16];
    const int swave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));

    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane % LPR;
    const int slot = lane / LPR;
    // byte offsets inside one wave iteration (rows it*kRowsPerWave ..
    // +kRowsPerWave-1): the iteration's base address is wave-uniform (scalar
    // registers), so the loop rewrites no per-lane address registers while
    // earlier loads are in flight
    const typename F::Lane g = F::lane(sub, ngroups, static_cast<uint32_t>(slot * row_bytes));
    // Loop control is 32-bit and scalar (the host keeps the iteration count
    // below 2^31): gfx9 has no 64-bit scalar compare, and a vector compare in
    // the loop would borrow registers that earlier memory operations still own.
    const int iter_bytes = kRowsPerWave * static_cast<int>(row_bytes);
    const int count = mt.count;
    const int niters = mt.it_begin[count];
    // A wave's iterations only move forward, so each side (the loads issued
    // ahead, the rows being finished) follows its own cursor over the
    // matrices and reads a table entry only when it crosses into the next
    // matrix (a scalar load from the argument segment).  Past the end a cursor
    // stays on the last matrix, with nothing left to load.
    struct LoadCursor {
        int mi, begin, end, tail;
        const uint8_t *w;
    };
    struct RowCursor {
        int mi, begin, end;
        int64_t n;
        YT *y;
        const float *r;
        YT *yg;
        int hl;
    };
    LoadCursor lc{0, 0, mt.it_begin[1], mt.tail_bytes[0], mt.w[0]};
    RowCursor rc{0, 0, mt.it_begin[1], mt.n[0], static_cast<YT *>(mt.y[0]), mt.r[0], static_cast<YT *>(mt.y_gate[0]),
                 mt.head_log2[0]};
    // moves the load cursor to iteration `it`: its byte offset in the
    // matrix, its byte count (0 past the end) and the matrix
    auto load_cursor = [&](int it, int64_t &off, int &nrec) -> const uint8_t * {
        while (it >= lc.end && lc.mi + 1 < count) {
            ++lc.mi;
            lc.begin = lc.end;
            lc.end = mt.it_begin[lc.mi + 1];
            lc.tail = mt.tail_bytes[lc.mi];
            lc.w = mt.w[lc.mi];
        }
        const int left = lc.end - it;
        off = static_cast<int64_t>(it - lc.begin) * iter_bytes;
        nrec = __builtin_amdgcn_readfirstlane(left > 1 ? iter_bytes : (left == 1 ? lc.tail : 0));
        // uniform by construction; said again so that the descriptor is built
        // in scalar registers whatever the compiler concluded across the joins
        return reinterpret_cast<const uint8_t *>(wave_uniform(reinterpret_cast<int64_t>(lc.w)));
    };
    // staged stream: iteration `it` into slot b of the wave's ring
    auto issue_stage = [&](int b, int it) {
        int64_t off;
        int nrec;
        const uint8_t *wbase = load_cursor(it, off, nrec);
#pragma unroll
        for (int m2 = 0; m2 < NMAT; ++m2) {
            stage_bytes<kIterBytes>(stream_rsrc((m2 == 0 ? wbase : wu) + off, nrec), &stage[b][m2][swave][0], lane);
        }
    };
    auto issue = [&](RowLoads<F, NMAT> (&b)[RPG], int it) {
        int64_t off;
        int nrec;
        const uint8_t *wbase = load_cursor(it, off, nrec);
#pragma unroll
        for (int q = 0; q < RPG; ++q) {
            const int sh = q * kRowsPerGroup * static_cast<int>(row_bytes);
            const int nq = nrec > sh ? nrec - sh : 0;
#pragma unroll
            for (int m2 = 0; m2 < NMAT; ++m2)
                F::issue(b[q].m[m2], stream_rsrc((m2 == 0 ? wbase : wu) + off + sh, nq), g);
        }
    };
    auto row_cursor = [&](int it) {
        while (it >= rc.end && rc.mi + 1 < count) {
            ++rc.mi;
            rc.begin = rc.end;
            rc.end = mt.it_begin[rc.mi + 1];
            rc.n = mt.n[rc.mi];
            rc.y = static_cast<YT *>(mt.y[rc.mi]);
            rc.r = mt.r[rc.mi];
            if constexpr (QG) {
                rc.yg = static_cast<YT *>(mt.y_gate[rc.mi]);
                rc.hl = mt.head_log2[rc.mi];
            }
        }
    };
    // Where row `row` of the current matrix goes: rows of head h are 2D
    // apart (D = 2^hl), the first D of them to y, the next D to the gate
    // output.  A plain matrix has hl so large that every row is in head 0's
    // first half: y + row.
    auto dest = [&](int64_t row) -> YT * {
        const int64_t d = int64_t{1} << rc.hl;
        const int64_t h = row >> (rc.hl + 1);
        const int64_t j = row - (h << (rc.hl + 1));
        return j < d ? rc.y + (h << rc.hl) + j : rc.yg + (h << rc.hl) + (j - d);
    };

    const int nwaves = static_cast<int>(gridDim.x) * kIterWaves;
    const int wave = static_cast<int>(threadIdx.x >> 6);
    const int it0 = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * kIterWaves + wave / TP);
    const int tile = __builtin_amdgcn_readfirstlane(wave % TP);

    // activations first, then the first rows' weights: waiting for the
    // activations (in issue order) then leaves the weight loads in flight
    constexpr int kXChunks = x_chunks(LPR, BLOCK);
    const int64_t xstride = static_cast<int64_t>(ngroups) * 64;
    XLoaded<kXChunks> xl[kTok];
#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        const XT *xt = x;
        if constexpr (kTok > 1) xt = x + (t < ntok ? t : ntok - 1) * xstride;
        xl[t] = load_x<BLOCK, kXChunks, XT>(xt, ngroups);
    }
    // keep the activation loads ahead of the weight loads (an empty asm with a
    // memory clobber: no instruction, only an ordering point for the compiler;
    // x is deliberately not __restrict__ so its loads cannot move across it)
    asm volatile("" ::: "memory");
    RowLoads<F, NMAT> buf[kStage ? 1 : NB][RPG];
    if constexpr (kStage) {
#pragma unroll
        for (int b = 0; b < kSlots; ++b) issue_stage(b, it0 + b * nwaves);
    } else {
#pragma unroll
        for (int b = 0; b + 1 < NB; ++b) issue(buf[b], it0 + b * nwaves);
    }

#pragma unroll
    for (int t = 0; t < kTok; ++t) {
        if (kTok == 1 || t < ntok) prepare_x<BLOCK, kXChunks>(xl[t], ngroups, xg + t * ngroups);
    }
    if constexpr (kStage) lds_barrier();  // the first iteration's loads stay in flight
    else __syncthreads();
    // the tokens of this wave (tokens past ntok repeat the last)
    int tok[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        tok[j] = 0;
        if constexpr (kTok > 1) {
            tok[j] = tile * MT + j;
            tok[j] = tok[j] < ntok ? tok[j] : ntok - 1;
        }
    }
    // token tiles: outputs of token tile*MT + j sit j*ystride after the
    // tile's first; nvalid of the tile's tokens exist
    const int64_t ystride = mt.n[0];
    const int nvalid = ntok - tile * MT;
    const int my_iters = (niters - it0 + nwaves - 1) / nwaves;

    // The row stream, on the integer path (EXACT false: src is the MT
    // tokens' activation registers) or the f32 path (EXACT true: src holds
    // MT pointers to the lane's group of activations, in registers or in
    // memory, and every weight is multiplied on its own).
    auto stream_rows = [&](auto exact_tag, const auto &src) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        // The loads are never inside a branch: at a control-flow join the wait
        // counters would have to assume the fewest loads in flight and drain the
        // prefetch.  Iterations past the end load nothing (0-byte descriptor).
        //
        // Results are not stored row by row: gfx9 counts stores with the loads,
        // and a store on some paths through the loop but not others makes the
        // wait counters drain loads still in flight.  Lane k of a row's lane group
        // keeps the group's k-th result of the current window of LPR rows (and
        // where it goes); the window is stored in one go when it is full (a wave
        // streaming fewer than LPR rows per group stores only after the loop).
        float yv[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) yv[j] = 0.0f;
        YT *yp = nullptr;
        const float *rp = nullptr;
        int win = 0;
        auto flush = [&]() {
            if (yp != nullptr) {
                if constexpr (RES) {
                    *yp = static_cast<YT>(rp != nullptr ? yv[0] + *rp : yv[0]);
                } else {
                    *yp = static_cast<YT>(yv[0]);
#pragma unroll
                    for (int j = 1; j < MT; ++j) {
                        if (j < nvalid) yp[j * ystride] = static_cast<YT>(yv[j]);
                    }
                }
            }
            yp = nullptr;
            win = 0;
        };
        // Finishes one wave iteration whose weights are in `rows` and whose
        // lane slot's first row is row0 of a matrix of nrows rows (output
        // ybase, residual rbase): the lane group's dot products, reduced, kept
        // for the window's store.
        auto finish_rows = [&](const RowLoads<F, NMAT> (&rows)[RPG], int64_t row0, int64_t nrows, YT *ybase,
                               const float *rbase) {
#pragma unroll
            for (int q = 0; q < RPG; ++q) {
                const int64_t row = row0 + q * kRowsPerGroup;
                const bool rok = row < nrows;
                const bool mine = sub == win;
                if constexpr (MT == 1) {
                    float acc[NMAT];
                    if constexpr (EXACT) lane_dot_exact(rows[q], g, src[0], rok && g.ok, 0.0f, acc);
                    else lane_dot(rows[q], g, src[0], rok && g.ok, acc);
                    if constexpr (SWIGLU && LPR == kWave) {
                        wave_sum_pair(acc[0], acc[1]);
                    } else {
#pragma unroll
                        for (int m2 = 0; m2 < NMAT; ++m2) acc[m2] = lane_group_sum<LPR>(acc[m2]);
                    }
                    const float out = SWIGLU ? silu(acc[0]) * acc[NMAT - 1] : acc[0];
                    yv[0] = mine ? out : yv[0];
                } else {
                    // one decode of the group for the wave's MT tokens
                    float acc[MT];
                    if constexpr (EXACT) F::dot_tokens_exact(rows[q].m[0], g, src, rok && g.ok, 0.0f, acc);
                    else F::dot_tokens(rows[q].m[0], g, src, rok && g.ok, acc);
#pragma unroll
                    for (int j = 0; j < MT; ++j) {
                        acc[j] = lane_group_sum<LPR>(acc[j]);
                        yv[j] = mine ? acc[j] : yv[j];
                    }
                }
                if constexpr (QG) yp = mine ? (rok ? dest(row) : nullptr) : yp;
                else if constexpr (kTok > 1) yp = mine ? (rok ? ybase + tile * MT * ystride + row : nullptr) : yp;
                else yp = mine ? (rok ? ybase + row : nullptr) : yp;
                if constexpr (RES) rp = mine ? (rbase != nullptr ? rbase + row : nullptr) : rp;
                if (++win == LPR) flush();
            }
        };
        // the same for iteration `cur` of the whole table (cursor over the matrices)
        auto finish = [&](const RowLoads<F, NMAT> (&rows)[RPG], int cur) {
            row_cursor(cur);
            finish_rows(rows, static_cast<int64_t>(cur - rc.begin) * kRowsPerWave + slot, rc.n, rc.y, rc.r);
        };
        // The sequencer issues from the oldest wave first, so with equal shares
        // the younger waves of a CU fall behind and finish alone, long after the
        // others.  Each wave therefore lowers its own priority as the share of its
        // iterations still to do drops (1/2, 1/4, 1/8): a wave that is behind
        // outranks the ones ahead of it, and the finish times close up.  kdone:
        // the wave's iterations finished so far.
        auto set_priority = [&](int kdone) {
            const int left = my_iters - kdone;
            if (2 * left > my_iters) __builtin_amdgcn_s_setprio(3);
            else if (4 * left > my_iters) __builtin_amdgcn_s_setprio(2);
            else if (8 * left > my_iters) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        };
        if constexpr (kStage) {
            // Staged: slot b of the ring holds iterations b, b + kSlots, ...
            // (in units of nwaves).  Each step waits for its slot's loads
            // (the other slots' kSlots - 1 iterations of loads, issued later,
            // stay in flight), reads the slot into registers, refills it with
            // the iteration kSlots ahead and decodes the registers meanwhile.
            auto fetch_slot = [&](RowLoads<F, NMAT> (&rows)[RPG], int b) {
    #pragma unroll
                for (int q = 0; q < RPG; ++q) {
    #pragma unroll
                    for (int m2 = 0; m2 < NMAT; ++m2)
                        F::fetch(rows[q].m[m2],
                                 lds_addr(&stage[b][m2][swave][0]) +
                                     static_cast<uint32_t>(q * kRowsPerGroup) * static_cast<uint32_t>(row_bytes),
                                 g);
                }
            };
            if (it0 < niters && !QG && count == 1) {
                // One matrix (the common call): the next load's byte offset
                // and the lane's row advance by constant strides, so a step
                // costs few scalar instructions (a vector instruction occupies
                // a SIMD for 4 cycles, and the scalar unit takes one
                // instruction per 4 cycles for all waves of a SIMD).
                const int64_t n0 = mt.n[0];
                YT *const y0 = static_cast<YT *>(mt.y[0]);
                const float *const r0 = mt.r[0];
                const uint8_t *const w0 = mt.w[0];
                const int tail = mt.tail_bytes[0];
                const int64_t lstep = static_cast<int64_t>(nwaves) * iter_bytes;
                int lit = it0 + kSlots * nwaves;  // iteration of the next load
                int64_t loff = static_cast<int64_t>(lit) * iter_bytes;
                int64_t row0 = static_cast<int64_t>(it0) * kRowsPerWave + slot;
                const int64_t rstep = static_cast<int64_t>(nwaves) * kRowsPerWave;
                int kdone = 0;
                for (;;) {
#pragma unroll
                    for (int b = 0; b < kSlots; ++b) {
                        set_priority(kdone);
                        wait_vm<kDma * NMAT * (kSlots - 1)>();
                        RowLoads<F, NMAT> rows[RPG];
                        fetch_slot(rows, b);
                        const int nrec = lit < niters - 1 ? iter_bytes : (lit == niters - 1 ? tail : 0);
#pragma unroll
                        for (int m2 = 0; m2 < NMAT; ++m2)
                            stage_bytes<kIterBytes>(stream_rsrc((m2 == 0 ? w0 : wu) + loff, nrec),
                                                    &stage[b][m2][swave][0], lane);
                        lit += nwaves;
                        loff += lstep;
                        finish_rows(rows, row0, n0, y0, r0);
                        row0 += rstep;
                        if (++kdone == my_iters) goto done;
                    }
                }
            } else if (it0 < niters) {
                int kdone = 0;
                for (int it = it0;; it += kSlots * nwaves) {
#pragma unroll
                    for (int b = 0; b < kSlots; ++b) {
                        const int cur = it + b * nwaves;
                        set_priority(kdone++);
                        wait_vm<kDma * NMAT * (kSlots - 1)>();
                        RowLoads<F, NMAT> rows[RPG];
                        fetch_slot(rows, b);
                        issue_stage(b, cur + kSlots * nwaves);
                        finish(rows, cur);
                        if (cur + nwaves >= niters) goto done;
                    }
                }
            }
        } else if (it0 < niters) {
            // The last iteration leaves both loops at once (goto): a break that
            // fell back to the outer loop's test would join the loop head with
            // loads of the unfinished unrolled pass still in flight, and the
            // wait counters would have to drain them there.
            int kdone = 0;
            for (int it = it0;; it += NB * nwaves) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int cur = it + b * nwaves;
                    set_priority(kdone++);
                    issue(buf[(b + NB - 1) % NB], cur + (NB - 1) * nwaves);
                    finish(buf[b], cur);
                    if (cur + nwaves >= niters) goto done;
                }
            }
        }
    done:
        flush();
    };

    XRegs xr[MT];
    uint32_t flagged = 0;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        load_xregs(xg[tok[j] * ngroups + g.j], xr[j]);
        flagged |= xr[j].inexact;
    }
    // A wave whose groups include a flagged one takes the f32 path for all
    // of them (the choice is per wave, so its loop has no branch on it).
    if (__builtin_amdgcn_ballot_w64(flagged != 0) == 0) {
        stream_rows(std::false_type{}, xr);
    } else {
        // the f32 path reads the lane's group of activations from memory
        // (the caches) for every row
        const XT *src[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) src[j] = x + tok[j] * xstride + 64 * g.j;
        stream_rows(std::true_type{}, src);
    }
}

// ------------------------------------------------------ 4096 < K <= 16384
// A row is split over S waves of the workgroup (S * 64 groups, wave s owns
// groups 64s .. 64s+63, one per lane, with its activation slice in registers);
// the workgroup streams R rows per block iteration, one per group of S waves.
// Each wave reduces its slice across its lanes and leaves the partial sum in
// LDS; every kFlush iterations (and at the end) a barrier, then one thread per
// row adds the S partials in slice order and stores the result, so the result
// does not depend on timing.  The partial buffer has two halves, so the next
// stretch of iterations writes while the last one is read.  res, if set, is
// added to each result (it may be y itself: each thread reads a row's
// residual before it writes that row).
//
// MT > 1: MT tokens (x [ntok][K], y [ntok][n], ntok <= MT; a missing token
// repeats the last and is not stored), each wave holding the activation
// registers of all of them and decoding each weight group once.
constexpr int kFlush = 8;

template <class F, typename XT, typename YT, int S, int R, bool SWIGLU, int NB, int MIN_WAVES, int MT = 1>
__global__ __launch_bounds__(64 * S * R, MIN_WAVES) void gemv_split_kernel(const uint8_t *__restrict__ w,
                                                                           const uint8_t *__restrict__ wu,
                                                                           const XT *x, YT *y,
                                                                           const float *res, int64_t n, int ngroups,
                                                                           int64_t row_bytes, int ntok) {
    static_assert(MT == 1 || !SWIGLU, "token tiles: plain GEMV");
    constexpr int BLOCK = 64 * S * R;
    constexpr int NMAT = SWIGLU ? 2 : 1;
    constexpr int NV = NMAT * MT;  // partial sums per row and slice
    extern __shared__ __align__(16) unsigned char smem[];
    XGroup *xg = reinterpret_cast<XGroup *>(smem);
    // [2][kFlush][R][S][NV]
    float *part = reinterpret_cast<float *>(smem + static_cast<size_t>(MT) * ngroups * sizeof(XGroup));
    // Single-token Q4_K rows stage each wave's slice (64 groups, 2304
    // contiguous bytes) through LDS, as gemv_kernel does: a ring of
    // kSlots = NB - 1 slices in flight per wave.
    constexpr bool kStage = F::kStaged && MT == 1 && !SWIGLU && Q4K_STAGE != 0;
    constexpr int kSlots = kStage ? NB - 1 : 1;
    constexpr int kSliceBytes = kWave * F::kGroupBytes;
    constexpr int kDma = stage_loads<kSliceBytes>();
    constexpr int kStageWaves = kStage ? S * R : 1;
    constexpr int kStageBytes = kStage ? kSliceBytes : 16;
    __shared__ __align__(16) uint8_t stage[kSlots][kStageWaves][kStageBytes];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int slice = wave % S;
    const int rslot = wave / S;
    const typename F::Lane g = F::lane(slice * kWave + lane, ngroups, 0u);
    // block iterations b = blockIdx.x + c * gridDim.x cover rows b*R .. b*R+R-1;
    // the host keeps gridDim.x <= the number of block iterations
    const int64_t nbi = (n + R - 1) / R;
    // the grid size once, in a scalar register (the loop would otherwise
    // reload it from the argument segment every iteration)
    const int nblk = __builtin_amdgcn_readfirstlane(static_cast<int>(gridDim.x));
    const int my_iters = static_cast<int>((nbi - 1 - blockIdx.x) / nblk) + 1;
    auto row_of = [&](int c, int r) -> int64_t {
        return (static_cast<int64_t>(blockIdx.x) + static_cast<int64_t>(c) * nblk) * R + r;
    };
    auto issue = [&](RowLoads<F, NMAT> &b, int c) {
        const int64_t row = row_of(c, rslot);
        const bool live = c < my_iters && row < n;
        issue_row(b, w, wu, live ? row * row_bytes : 0, live ? static_cast<int>(row_bytes) : 0, g);
    };
    // staged: the wave's slice of iteration c into slot b of its ring
    auto slot = [&](int b) -> uint8_t * { return &stage[b][wave][0]; };
    auto issue_stage = [&](int b, int c) {
        const int64_t row = row_of(c, rslot);
        const bool live = c < my_iters && row < n;
        const int64_t sb = static_cast<int64_t>(slice) * kSliceBytes;
        const int64_t left = row_bytes - sb;
        const int nrec = __builtin_amdgcn_readfirstlane(
            live ? static_cast<int>(left < kSliceBytes ? (left > 0 ? left : 0) : kSliceBytes) : 0);
        const uint8_t *base =
            reinterpret_cast<const uint8_t *>(wave_uniform(reinterpret_cast<int64_t>(w + (live ? row * row_bytes + sb : 0))));
        stage_bytes<kSliceBytes>(stream_rsrc(base, nrec), slot(b), lane);
    };
    // the lane's byte offsets inside its slice (its validity and pair
    // selection come from g)
    const typename F::Lane gs = F::lane(lane, kWave, 0u);

    constexpr int kXChunks = x_chunks(S * kWave, BLOCK);
    const int64_t xstride = static_cast<int64_t>(ngroups) * 64;
    XLoaded<kXChunks> xl[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const XT *xt = x;
        if constexpr (MT > 1) xt = x + (t < ntok ? t : ntok - 1) * xstride;
        xl[t] = load_x<BLOCK, kXChunks, XT>(xt, ngroups);
    }
    asm volatile("" ::: "memory");
    RowLoads<F, NMAT> buf[kStage ? 1 : NB];
    if constexpr (kStage) {
#pragma unroll
        for (int b = 0; b < kSlots; ++b) issue_stage(b, b);
    } else {
#pragma unroll
        for (int b = 0; b + 1 < NB; ++b) issue(buf[b], b);
    }
    auto barrier = [&]() {
        if constexpr (kStage) lds_barrier();
        else __syncthreads();
    };

    __shared__ int inexact;
    if (threadIdx.x == 0) inexact = 0;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (MT == 1 || t < ntok) prepare_x<BLOCK, kXChunks>(xl[t], ngroups, xg + t * ngroups);
    }
    barrier();
    int tok[MT];
    uint32_t flagged = 0;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        tok[t] = MT == 1 ? 0 : (t < ntok ? t : ntok - 1);
        flagged |= g.ok ? xg[tok[t] * ngroups + g.j].inexact : 0u;
    }
    // The loop below has barriers, so the choice of path is made once for the
    // whole workgroup: the f32 path if any wave's slice holds a flagged group.
    if (__builtin_amdgcn_ballot_w64(flagged != 0) != 0 && lane == 0) inexact = 1;
    barrier();

    // EXACT false: src is the MT tokens' activation registers; EXACT true:
    // MT pointers to the lane's group of activations (registers or memory).
    auto stream_rows = [&](auto exact_tag, const auto &src) {
        constexpr bool EXACT = decltype(exact_tag)::value;
        // f32 path: each row's reads wait for the previous row's sums (the
        // unrolled rows would otherwise all hold their activations at once)
        float chain = 0.0f;
        // the lane's share of iteration cur, reduced into LDS; every kFlush
        // iterations (and at the end) the rows' slices are added and stored
        auto finish = [&](const RowLoads<F, NMAT> &rows, int cur) {
            float acc[NV];
            if constexpr (MT == 1) {
                if constexpr (EXACT) lane_dot_exact(rows, g, src[0], g.ok, chain, acc);
                else lane_dot(rows, g, src[0], g.ok, acc);
            } else {
                float at[MT];
                if constexpr (EXACT) F::dot_tokens_exact(rows.m[0], g, src, g.ok, chain, at);
                else F::dot_tokens(rows.m[0], g, src, g.ok, at);
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = at[t];
            }
            if constexpr (EXACT) chain = acc[NV - 1];
            const int d = cur % kFlush;
            const int half = (cur / kFlush) & 1;
            float *pp = part + (((half * kFlush + d) * R + rslot) * S + slice) * NV;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                acc[v] = lane_group_sum<kWave>(acc[v]);
                if (lane == 0) pp[v] = acc[v];
            }
            if (d == kFlush - 1 || cur + 1 == my_iters) {
                barrier();
                const int t = static_cast<int>(threadIdx.x);
                if (t < (d + 1) * R) {
                    const int dd = t / R;
                    const int r = t % R;
                    const int64_t row = row_of(cur - d + dd, r);
                    if (row < n) {
                        const float *q = part + ((half * kFlush + dd) * R + r) * S * NV;
                        float sum[NV];
#pragma unroll
                        for (int v = 0; v < NV; ++v) sum[v] = q[v];
#pragma unroll
                        for (int s = 1; s < S; ++s) {
#pragma unroll
                            for (int v = 0; v < NV; ++v) sum[v] += q[s * NV + v];
                        }
                        if constexpr (MT == 1) {
                            const float v = SWIGLU ? silu(sum[0]) * sum[NV - 1] : sum[0];
                            y[row] = static_cast<YT>(res != nullptr ? v + res[row] : v);
                        } else {
#pragma unroll
                            for (int j = 0; j < MT; ++j) {
                                if (j < ntok) y[j * n + row] = static_cast<YT>(sum[j]);
                            }
                        }
                    }
                }
            }
        };
        // priority falls with the share of iterations left, as in gemv_kernel
        auto set_priority = [&](int c) {
            const int left = my_iters - c;
            if (4 * left > 3 * my_iters) __builtin_amdgcn_s_setprio(3);
            else if (4 * left > 2 * my_iters) __builtin_amdgcn_s_setprio(2);
            else if (4 * left > my_iters) __builtin_amdgcn_s_setprio(1);
            else __builtin_amdgcn_s_setprio(0);
        };
        if constexpr (kStage) {
            // slot b holds iterations b, b + kSlots, ...: wait for its loads
            // (the other slots' stay in flight), read it, refill it with the
            // wave's iteration kSlots ahead, decode the registers meanwhile
            for (int c = 0; c < my_iters; c += kSlots) {
                set_priority(c);
#pragma unroll
                for (int b = 0; b < kSlots; ++b) {
                    const int cur = c + b;
                    wait_vm<kDma * (kSlots - 1)>();
                    RowLoads<F, NMAT> rows;
                    F::fetch(rows.m[0], lds_addr(slot(b)), gs);
                    issue_stage(b, cur + kSlots);
                    finish(rows, cur);
                    if (cur + 1 >= my_iters) break;
                }
            }
        } else {
            for (int c = 0; c < my_iters; c += NB) {
                set_priority(c);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int cur = c + b;
                    // the f32 path loads each row just before it is used, after the
                    // previous row's result (few registers: it is a fallback)
                    if constexpr (EXACT) issue(buf[b], opaque_int_after(cur, chain));
                    else issue(buf[(b + NB - 1) % NB], cur + NB - 1);
                    finish(buf[b], cur);
                    if (cur + 1 >= my_iters) break;
                }
            }
        }
    };

    if (inexact == 0) {
        XRegs xr[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) load_xregs(xg[tok[t] * ngroups + g.j], xr[t]);
        stream_rows(std::false_type{}, xr);
    } else {
        const XT *src[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) src[t] = x + tok[t] * xstride + 64 * g.j;
        stream_rows(std::true_type{}, src);
    }
}

// Any K: one wave per row, each lane dequantizes four weights at a time in f32
// and accumulates x * w with FMA; activations read straight from memory.
template <typename XT, typename YT, bool SWIGLU>
__global__ __launch_bounds__(256) void gemv_generic_kernel(const uint8_t *__restrict__ w,
                                                           const uint8_t *__restrict__ wu,
                                                           const XT *__restrict__ x, YT *y,
                                                           const float *res, int64_t n, int64_t k, int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
    const int64_t quads = k / 4;
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); row < n; row += nwaves) {
        float acc[2] = {0.0f, 0.0f};
#pragma unroll
        for (int mat = 0; mat < (SWIGLU ? 2 : 1); ++mat) {
            const uint8_t *r = (mat == 0 ? w : wu) + row * row_bytes;
            for (int64_t t = lane; t < quads; t += 64) {
                const int64_t blk = t >> 6;
                const int e0 = static_cast<int>(t & 63) * 4;
                const uint8_t *b = r + blk * kBlockBytes;
                const uint4 hdr = *reinterpret_cast<const uint4 *>(b);
                const int g = e0 >> 6;
                const int rr = e0 & 63;
                const uint32_t codes = *reinterpret_cast<const uint32_t *>(b + 16 + 32 * g + (rr & 31));
                const uint32_t nib = (rr < 32) ? (codes & 0x0f0f0f0fu) : ((codes >> 4) & 0x0f0f0f0fu);
                int sc, m;
                scale_min(hdr.y, hdr.z, hdr.w, 2 * g + (rr >> 5), sc, m);
                const float dl = half_bits_to_float(hdr.x) * static_cast<float>(sc);
                const float ml = half_bits_to_float(hdr.x >> 16) * static_cast<float>(m);
                const XT *xp = x + 4 * t;
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    const float wv = dl * static_cast<float>((nib >> (8 * b4)) & 0xffu) - ml;
                    acc[mat] = fmaf(wv, static_cast<float>(xp[b4]), acc[mat]);
                }
            }
            acc[mat] = group_sum<64>(acc[mat]);
        }
        if (lane == 0) {
            const float v = SWIGLU ? silu(acc[0]) * acc[1] : acc[0];
            y[row] = static_cast<YT>(res != nullptr ? v + res[row] : v);
        }
    }
}

// Q8_0, any K % 32 == 0 and any 2-byte aligned matrix: one wave per row, each
// lane takes whole blocks (16-bit loads) and accumulates d*q*x with FMA.
__global__ __launch_bounds__(256) void q8_0_generic_kernel(const uint8_t *__restrict__ w,
                                                           const float *__restrict__ x, float *y, const float *res,
                                                           int64_t n, int64_t k, int64_t row_bytes) {
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * 4;
    const int64_t nblocks = k / Q8_0Format::kBlockWeights;
    for (int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); row < n; row += nwaves) {
        float acc = 0.0f;
        for (int64_t b = lane; b < nblocks; b += 64) {
            const uint16_t *blk = reinterpret_cast<const uint16_t *>(w + row * row_bytes + b * Q8_0Format::kBlockBytes);
            const float d = half_bits_to_float(blk[0]);
            const float *xp = x + b * Q8_0Format::kBlockWeights;
#pragma unroll
            for (int h = 0; h < 16; ++h) {
                const uint32_t pair = blk[1 + h];
                const float w0 = d * static_cast<float>(static_cast<int8_t>(pair & 0xffu));
                const float w1 = d * static_cast<float>(static_cast<int8_t>(pair >> 8));
                acc = fmaf(w0, xp[2 * h], acc);
                acc = fmaf(w1, xp[2 * h + 1], acc);
            }
        }
        acc = group_sum<64>(acc);
        if (lane == 0) y[row] = res != nullptr ? acc + res[row] : acc;
    }
}

namespace {

constexpr int kMaxDevices = 64;

template <typename Kernel>
int resident_blocks_per_cu(Kernel kern, int block, size_t lds, std::atomic<int> *cache) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, block, lds) != hipSuccess || nb < 1) nb = 1;
    cache[dev].store(nb, std::memory_order_relaxed);
    return nb;
}

// One launch of the batch-1 kernel over `count` matrices (all with k columns).
template <class F, typename XT, typename YT, int LPR, bool SWIGLU, bool RES, int NB, int BLOCK, int MIN_WAVES,
          int RPG, bool QG = false>
hipError_t launch_fast_kernel(const GemvJob *jobs, int count, const uint8_t *wu, const void *x, int64_t k,
                              hipStream_t stream) {
    auto kern = gemv_kernel<F, XT, YT, LPR, SWIGLU, RES, NB, BLOCK, MIN_WAVES, RPG, QG>;
    const int ngroups = static_cast<int>(k / 64);
    const int64_t row_bytes = F::row_bytes(k);
    const size_t lds = static_cast<size_t>(ngroups) * sizeof(XGroup);
    static std::atomic<int> cache[kMaxDevices];
    const int per_cu = resident_blocks_per_cu(kern, BLOCK, lds, cache);
    constexpr int kRowsPerWave = RPG * (kWave / LPR);
    MatTable mt{};
    mt.count = count;
    int64_t total = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t iters = (jobs[i].n + kRowsPerWave - 1) / kRowsPerWave;
        mt.w[i] = jobs[i].w;
        mt.y[i] = jobs[i].y;
        mt.r[i] = jobs[i].r;
        mt.n[i] = jobs[i].n;
        mt.y_gate[i] = jobs[i].y_gate;
        mt.head_log2[i] = jobs[i].head_log2;
        mt.it_begin[i] = static_cast<int>(total);
        mt.tail_bytes[i] = static_cast<int>((jobs[i].n - (iters - 1) * kRowsPerWave) * row_bytes);
        total += iters;
    }
    // 32-bit loop control in the kernel (unreachable: 2^30 iterations are
    // terabytes of weights)
    if (total >= (int64_t{1} << 30)) return hipErrorInvalidValue;
    for (int i = count; i <= kMaxMats; ++i) mt.it_begin[i] = static_cast<int>(total);
    const int64_t need = (total + BLOCK / kWave - 1) / (BLOCK / kWave);
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    const int grid = static_cast<int>(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(BLOCK), lds, stream, mt, wu, static_cast<const XT *>(x), ngroups,
                       row_bytes, 1);
    return hipGetLastError();
}

template <class F, typename XT, typename YT, int S, int R, bool SWIGLU, int NB, int MIN_WAVES, int MT = 1>
hipError_t launch_split(const uint8_t *w, const uint8_t *wu, const void *x, const float *r, void *y, int64_t n,
                        int64_t k, hipStream_t stream, int ntok = 1) {
    auto kern = gemv_split_kernel<F, XT, YT, S, R, SWIGLU, NB, MIN_WAVES, MT>;
    constexpr int BLOCK = 64 * S * R;
    const int ngroups = static_cast<int>(k / 64);
    const size_t lds = static_cast<size_t>(MT) * ngroups * sizeof(XGroup) +
                       sizeof(float) * 2 * kFlush * R * S * (SWIGLU ? 2 : 1) * MT;
    static std::atomic<int> cache[kMaxDevices];
    const int per_cu = resident_blocks_per_cu(kern, BLOCK, lds, cache);
    const int64_t need = (n + R - 1) / R;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    const int grid = static_cast<int>(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(BLOCK), lds, stream, w, wu, static_cast<const XT *>(x),
                       static_cast<YT *>(y), r, n, ngroups, F::row_bytes(k), ntok);
    return hipGetLastError();
}

// One launch of the token-tile kernel: m tokens (MT * (TP - 1) < m <= MT * TP)
// against one matrix of n rows.
template <typename XT, typename YT, int LPR, int MT, int TP, int NB, int BLOCK, int MIN_WAVES>
hipError_t launch_tokens_kernel(const uint8_t *w, const void *x, void *y, int m, int64_t n, int64_t k,
                                hipStream_t stream) {
    auto kern = gemv_kernel<Q4KFormat, XT, YT, LPR, false, false, NB, BLOCK, MIN_WAVES, 1, false, MT, TP>;
    const int ngroups = static_cast<int>(k / 64);
    const int64_t row_bytes = Q4KFormat::row_bytes(k);
    // every token's activation groups; the occupancy query takes the largest
    const size_t lds = static_cast<size_t>(m) * ngroups * sizeof(XGroup);
    static std::atomic<int> cache[kMaxDevices];
    const int per_cu = resident_blocks_per_cu(kern, BLOCK, static_cast<size_t>(MT * TP) * ngroups * sizeof(XGroup),
                                              cache);
    constexpr int kRowsPerWave = kWave / LPR;
    constexpr int kIterWaves = BLOCK / kWave / TP;
    const int64_t iters = (n + kRowsPerWave - 1) / kRowsPerWave;
    if (iters >= (int64_t{1} << 30)) return hipErrorInvalidValue;
    MatTable mt{};
    mt.count = 1;
    mt.w[0] = w;
    mt.y[0] = y;
    mt.n[0] = n;
    mt.head_log2[0] = GemvJob::kPlainHead;
    for (int i = 1; i <= kMaxMats; ++i) mt.it_begin[i] = static_cast<int>(iters);
    mt.tail_bytes[0] = static_cast<int>((n - (iters - 1) * kRowsPerWave) * row_bytes);
    const int64_t need = (iters + kIterWaves - 1) / kIterWaves;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    const int grid = static_cast<int>(need < cap ? need : cap);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(BLOCK), lds, stream, mt, nullptr, static_cast<const XT *>(x), ngroups,
                       row_bytes, m);
    return hipGetLastError();
}

// Launch shape of the token-tile kernel: two tokens' activation registers
// (102 VGPRs) per wave.
#ifndef Q4K_TOK_BLOCK
#define Q4K_TOK_BLOCK 768
#endif
#ifndef Q4K_TOK_MINW
#define Q4K_TOK_MINW 3
#endif
#ifndef Q4K_TOK_NB
#define Q4K_TOK_NB 2
#endif

template <typename XT, typename YT, int LPR>
hipError_t dispatch_tokens_lpr(const uint8_t *w, const void *x, void *y, int m, int64_t n, int64_t k,
                               hipStream_t stream) {
    constexpr int B = Q4K_TOK_BLOCK, W = Q4K_TOK_MINW, NB = Q4K_TOK_NB;
    if (m <= 2) return launch_tokens_kernel<XT, YT, LPR, 2, 1, NB, B, W>(w, x, y, m, n, k, stream);
    return launch_tokens_kernel<XT, YT, LPR, 2, 2, NB, B, W>(w, x, y, m, n, k, stream);
}

// K-split shapes for two tokens (4096 < K <= 16384)
#ifndef Q4K_TOK_SPLIT_R
#define Q4K_TOK_SPLIT_R 4
#endif
#ifndef Q4K_TOK_SPLIT_NB
#define Q4K_TOK_SPLIT_NB 2
#endif
#ifndef Q4K_TOK_SPLIT_MINW
#define Q4K_TOK_SPLIT_MINW 2
#endif

template <typename XT, typename YT>
hipError_t dispatch_tokens(const uint8_t *w, const void *x, void *y, int m, int64_t n, int64_t k,
                           hipStream_t stream) {
    const int64_t ngroups = k / 64;
    if (ngroups > 64) {
        constexpr int R = Q4K_TOK_SPLIT_R, NB = Q4K_TOK_SPLIT_NB, W = Q4K_TOK_SPLIT_MINW;
        if (ngroups <= 128)
            return launch_split<Q4KFormat, XT, YT, 2, R, false, NB, W, 2>(w, nullptr, x, nullptr, y, n, k, stream, m);
        if (ngroups <= 192)
            return launch_split<Q4KFormat, XT, YT, 3, R, false, NB, W, 2>(w, nullptr, x, nullptr, y, n, k, stream, m);
        // four slices: two rows per workgroup keep it at 512 threads (registers)
        return launch_split<Q4KFormat, XT, YT, 4, 2, false, NB, W, 2>(w, nullptr, x, nullptr, y, n, k, stream, m);
    }
    if (ngroups <= 4) return dispatch_tokens_lpr<XT, YT, 4>(w, x, y, m, n, k, stream);
    if (ngroups <= 8) return dispatch_tokens_lpr<XT, YT, 8>(w, x, y, m, n, k, stream);
    if (ngroups <= 16) return dispatch_tokens_lpr<XT, YT, 16>(w, x, y, m, n, k, stream);
    if (ngroups <= 32) return dispatch_tokens_lpr<XT, YT, 32>(w, x, y, m, n, k, stream);
    return dispatch_tokens_lpr<XT, YT, 64>(w, x, y, m, n, k, stream);
}

template <class F, typename XT, typename YT, int LPR, bool SWIGLU, int NB, int BLOCK, int MIN_WAVES, int RPG = 1>
hipError_t launch_fast(const GemvJob *jobs, int count, const uint8_t *wu, const void *x, int64_t k,
                       hipStream_t stream) {
    bool res = false, qg = false;
    for (int i = 0; i < count; ++i) {
        res = res || jobs[i].r != nullptr;
        qg = qg || jobs[i].y_gate != nullptr;
    }
    if constexpr (std::is_same_v<XT, float> && std::is_same_v<YT, float> && !SWIGLU) {
        // a per-head de-interleave comes only from the multi-matrix call,
        // which has no residual
        if (qg) {
            return launch_fast_kernel<F, XT, YT, LPR, SWIGLU, false, NB, BLOCK, MIN_WAVES, RPG, true>(jobs, count, wu, x,
                                                                                                    k, stream);
        }
        if (res) {
            return launch_fast_kernel<F, XT, YT, LPR, SWIGLU, true, NB, BLOCK, MIN_WAVES, RPG>(jobs, count, wu, x, k,
                                                                                              stream);
        }
    }
    return launch_fast_kernel<F, XT, YT, LPR, SWIGLU, false, NB, BLOCK, MIN_WAVES, RPG>(jobs, count, wu, x, k, stream);
}

template <class F, typename XT, typename YT, bool SWIGLU>
hipError_t launch_generic(const uint8_t *w, const uint8_t *wu, const void *x, const float *r, void *y, int64_t n,
                          int64_t k, hipStream_t stream) {
    const int64_t need = (n + 3) / 4;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
    const int grid = static_cast<int>(need < cap ? need : cap);
    if constexpr (std::is_base_of_v<Q8_0Format, F>) {
        static_assert(!SWIGLU && std::is_same_v<XT, float> && std::is_same_v<YT, float>, "Q8_0: f32 GEMV only");
        hipLaunchKernelGGL(q8_0_generic_kernel, dim3(grid), dim3(256), 0, stream, w, static_cast<const float *>(x),
                           static_cast<float *>(y), r, n, k, F::row_bytes(k));
    } else {
        hipLaunchKernelGGL((gemv_generic_kernel<XT, YT, SWIGLU>), dim3(grid), dim3(256), 0, stream, w, wu,
                           static_cast<const XT *>(x), static_cast<YT *>(y), r, n, k, F::row_bytes(k));
    }
    return hipGetLastError();
}

// Launch shapes: threads per block, minimum resident waves per SIMD (the
// register budget) and row buffers per wave.  Streams of several MB run best
// as one 1024-thread block per CU (4 waves per SIMD; more resident waves
// measured slower); small matrices, which finish in a few microseconds, start
// faster with 256-thread blocks (less activation preparation per block, more
// blocks).
#ifndef Q4K_LARGE_BLOCK
#define Q4K_LARGE_BLOCK 1024
#endif
// rows of at most 1024 weights (16 lanes per row, four rows per wave
// iteration) stream faster from smaller workgroups: 512 threads for Q4_K,
// 256 for Q8_0 (measured on the 0.8B lm_head, 4-5 % each)
#ifndef Q4K_LARGE_BLOCK_SHORT
#define Q4K_LARGE_BLOCK_SHORT 512
#endif
#ifndef Q8_0_LARGE_BLOCK_SHORT
#define Q8_0_LARGE_BLOCK_SHORT 256
#endif
#ifndef Q4K_LARGE_MINW
#define Q4K_LARGE_MINW 4
#endif
#ifndef Q4K_LARGE_NB
#define Q4K_LARGE_NB 2
#endif
#ifndef Q4K_LARGE_RPG
#define Q4K_LARGE_RPG 1
#endif
#ifndef Q4K_SMALL_BLOCK
#define Q4K_SMALL_BLOCK 256
#endif
#ifndef Q4K_SMALL_MINW
#define Q4K_SMALL_MINW 3
#endif
#ifndef Q4K_SMALL_NB
#define Q4K_SMALL_NB 2
#endif
#ifndef Q4K_SWIGLU_WIDE_ROWS
#define Q4K_SWIGLU_WIDE_ROWS 8192
#endif
#ifndef Q4K_SWIGLU_WIDE_BLOCK
#define Q4K_SWIGLU_WIDE_BLOCK 768
#endif
#ifndef Q4K_SWIGLU_WIDE_MINW
#define Q4K_SWIGLU_WIDE_MINW 3
#endif
#ifndef Q4K_SWIGLU_BLOCK
#define Q4K_SWIGLU_BLOCK 512
#endif
#ifndef Q4K_SWIGLU_MINW
#define Q4K_SWIGLU_MINW 2
#endif
#ifndef Q4K_SWIGLU_NB
#define Q4K_SWIGLU_NB 2
#endif
#ifndef Q4K_SPLIT_NB
#define Q4K_SPLIT_NB 3
#endif
// Single-token Q4_K streams read through an LDS ring of this many iterations
// per wave (one slot per matrix each, 2304 bytes per 64 groups); Q8_0 keeps
// the register buffers above.  Deeper rings measured slower wherever they fit
// (the 9B lm_head: 85.3, 87.9, 88.9 us for 1, 2, 3 slots; the 9B down: 8.4 us
// with 1 slot, 8.6 with 2, 9.3 with 3): more loads queued per CU do not
// stream faster.  The K-split ring and the activation groups must fit the 160
// KB of LDS: two slices per row (16 waves, K <= 8192), three (12 waves,
// K <= 12288) and four (16 waves, K <= 16384).
#ifndef Q4K_LARGE_SLOTS
#define Q4K_LARGE_SLOTS 1
#endif
#ifndef Q4K_SMALL_SLOTS
#define Q4K_SMALL_SLOTS 1
#endif
#ifndef Q4K_SWIGLU_SLOTS
#define Q4K_SWIGLU_SLOTS 1
#endif
#ifndef Q4K_SPLIT2_SLOTS
#define Q4K_SPLIT2_SLOTS 3
#endif
#ifndef Q4K_SPLIT3_SLOTS
#define Q4K_SPLIT3_SLOTS 1
#endif
#ifndef Q4K_SPLIT4_SLOTS
#define Q4K_SPLIT4_SLOTS 2
#endif
// matrices below this many bytes use the small launch shape
#ifndef Q4K_SMALL_BYTES
#define Q4K_SMALL_BYTES (8 << 20)
#endif

template <class F, typename XT, typename YT, int LPR, bool SWIGLU>
hipError_t dispatch_lpr(const GemvJob *jobs, int count, const uint8_t *wu, const void *x, int64_t k,
                        hipStream_t stream) {
    // staged streams: NB - 1 = slots of the LDS ring
    constexpr bool kStaged = F::kStaged;
    if constexpr (SWIGLU) {
        constexpr int NB = kStaged ? 1 + Q4K_SWIGLU_SLOTS : Q4K_SWIGLU_NB;
        if constexpr (LPR == 64) {
            // many rows of a whole wave each: one 12-wave workgroup per CU
            // (2 % faster at 12288 rows; slower with few rows, where more,
            // smaller workgroups spread the rows better)
            int64_t rows = 0;
            for (int i = 0; i < count; ++i) rows += jobs[i].n;
            if (rows >= Q4K_SWIGLU_WIDE_ROWS) {
                return launch_fast<F, XT, YT, LPR, true, NB, Q4K_SWIGLU_WIDE_BLOCK, Q4K_SWIGLU_WIDE_MINW>(
                    jobs, count, wu, x, k, stream);
            }
        }
        return launch_fast<F, XT, YT, LPR, true, NB, Q4K_SWIGLU_BLOCK, Q4K_SWIGLU_MINW>(jobs, count, wu, x, k, stream);
    } else {
        int64_t bytes = 0;
        for (int i = 0; i < count; ++i) bytes += jobs[i].n * F::row_bytes(k);
        if (bytes < Q4K_SMALL_BYTES) {
            constexpr int NB = kStaged ? 1 + Q4K_SMALL_SLOTS : Q4K_SMALL_NB;
            return launch_fast<F, XT, YT, LPR, false, NB, Q4K_SMALL_BLOCK, Q4K_SMALL_MINW>(jobs, count, wu, x, k, stream);
        }
        constexpr int kShort = std::is_base_of_v<Q8_0Format, F> ? Q8_0_LARGE_BLOCK_SHORT : Q4K_LARGE_BLOCK_SHORT;
        constexpr int kBlock = LPR <= 16 ? kShort : Q4K_LARGE_BLOCK;
        constexpr int NB = kStaged ? 1 + Q4K_LARGE_SLOTS : Q4K_LARGE_NB;
        return launch_fast<F, XT, YT, LPR, false, NB, kBlock, Q4K_LARGE_MINW, Q4K_LARGE_RPG>(jobs, count, wu, x, k,
                                                                                           stream);
    }
}

// Rows wider than 4096 weights: one launch per matrix.
template <class F, typename XT, typename YT, bool SWIGLU>
hipError_t dispatch_wide(const GemvJob &j, const uint8_t *wu, const void *x, int64_t k, hipStream_t stream) {
    const int64_t ngroups = k / 64;
    // split rows: S waves per row; two matrices' row buffers need more
    // registers, so the SwiGLU shapes keep fewer rows per workgroup
    constexpr int NB = Q4K_SPLIT_NB;
    if constexpr (SWIGLU) {
        if (ngroups <= 128) return launch_split<F, XT, YT, 2, 4, true, NB, 2>(j.w, wu, x, j.r, j.y, j.n, k, stream);
        if (ngroups <= 192) return launch_split<F, XT, YT, 3, 4, true, NB, 3>(j.w, wu, x, j.r, j.y, j.n, k, stream);
        if (ngroups <= 256) return launch_split<F, XT, YT, 4, 2, true, NB, 2>(j.w, wu, x, j.r, j.y, j.n, k, stream);
    } else {
        constexpr bool kStaged = F::kStaged;
        constexpr int NB2 = kStaged ? 1 + Q4K_SPLIT2_SLOTS : NB;
        constexpr int NB3 = kStaged ? 1 + Q4K_SPLIT3_SLOTS : NB;
        constexpr int NB4 = kStaged ? 1 + Q4K_SPLIT4_SLOTS : NB;
        if (ngroups <= 128) return launch_split<F, XT, YT, 2, 8, false, NB2, 4>(j.w, wu, x, j.r, j.y, j.n, k, stream);
        if (ngroups <= 192) return launch_split<F, XT, YT, 3, 4, false, NB3, 3>(j.w, wu, x, j.r, j.y, j.n, k, stream);
        if (ngroups <= 256) return launch_split<F, XT, YT, 4, 4, false, NB4, 4>(j.w, wu, x, j.r, j.y, j.n, k, stream);
    }
    // beyond K = 16384: the plain kernel
    return launch_generic<F, XT, YT, SWIGLU>(j.w, wu, x, j.r, j.y, j.n, k, stream);
}

template <class F, typename XT, typename YT, bool SWIGLU>
hipError_t dispatch_short(const GemvJob *jobs, int count, const uint8_t *wu, const void *x, int64_t k,
                          hipStream_t stream) {
    const int64_t ngroups = k / 64;
    if (ngroups <= 4) return dispatch_lpr<F, XT, YT, 4, SWIGLU>(jobs, count, wu, x, k, stream);
    if (ngroups <= 8) return dispatch_lpr<F, XT, YT, 8, SWIGLU>(jobs, count, wu, x, k, stream);
    if (ngroups <= 16) return dispatch_lpr<F, XT, YT, 16, SWIGLU>(jobs, count, wu, x, k, stream);
    if (ngroups <= 32) return dispatch_lpr<F, XT, YT, 32, SWIGLU>(jobs, count, wu, x, k, stream);
    return dispatch_lpr<F, XT, YT, 64, SWIGLU>(jobs, count, wu, x, k, stream);
}

template <class F, typename XT, typename YT, bool SWIGLU>
hipError_t dispatch(const GemvJob *jobs, int count, const uint8_t *wu, const void *x, int64_t k,
                    hipStream_t stream) {
    if (k <= 4096) return dispatch_short<F, XT, YT, SWIGLU>(jobs, count, wu, x, k, stream);
    for (int i = 0; i < count; ++i) {
        const hipError_t e = dispatch_wide<F, XT, YT, SWIGLU>(jobs[i], wu, x, k, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv(const uint8_t *w, const uint8_t *w_up, const float *x, const float *r, float *y, int64_t n,
                       int64_t k, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const GemvJob job{w, y, r, n};
    return launch_gemv_multi(&job, 1, w_up, x, k, stream);
}

hipError_t launch_gemv_multi(const GemvJob *jobs, int count, const uint8_t *w_up, const float *x, int64_t k,
                             hipStream_t stream) {
    if (count < 0 || count > kMaxMats) return hipErrorInvalidValue;
    // empty matrices launch nothing; k == 0 is an empty sum (plus any residual)
    GemvJob live[kMaxMats];
    int nlive = 0;
    for (int i = 0; i < count; ++i) {
        if (jobs[i].n == 0) continue;
        if (k == 0) {
            float *y = static_cast<float *>(jobs[i].y);
            const bool split = jobs[i].y_gate != nullptr;
            const int64_t ny = split ? jobs[i].n / 2 : jobs[i].n;
            hipError_t e = jobs[i].r != nullptr ? launch_copy(y, jobs[i].r, ny, stream)
                                                : launch_fill_zero(y, ny, stream);
            if (e == hipSuccess && split) e = launch_fill_zero(static_cast<float *>(jobs[i].y_gate), ny, stream);
            if (e != hipSuccess) return e;
            continue;
        }
        live[nlive++] = jobs[i];
    }
    if (nlive == 0) return hipSuccess;
    if (w_up != nullptr) return dispatch<Q4KFormat, float, float, true>(live, nlive, w_up, x, k, stream);
    return dispatch<Q4KFormat, float, float, false>(live, nlive, nullptr, x, k, stream);
}

hipError_t launch_gemv_dt(const uint8_t *w, const void *x, bool x_f16, void *y, bool y_f16, int64_t n, int64_t k,
                          hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (k == 0) {
        return y_f16 ? launch_fill_zero_f16(static_cast<_Float16 *>(y), n, stream)
                     : launch_fill_zero(static_cast<float *>(y), n, stream);
    }
    const GemvJob job{w, y, nullptr, n};
    if (x_f16 && y_f16) return dispatch<Q4KFormat, _Float16, _Float16, false>(&job, 1, nullptr, x, k, stream);
    if (x_f16) return dispatch<Q4KFormat, _Float16, float, false>(&job, 1, nullptr, x, k, stream);
    if (y_f16) return dispatch<Q4KFormat, float, _Float16, false>(&job, 1, nullptr, x, k, stream);
    return dispatch<Q4KFormat, float, float, false>(&job, 1, nullptr, x, k, stream);
}

hipError_t launch_gemv_tokens(const uint8_t *w, const void *x, bool x_f16, void *y, bool y_f16, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
    if (m < 2 || m > (k <= kTokensMaxK ? kTokensMax : 2) || k <= 0 || k > kTokensSplitMaxK || n == 0) {
        return hipErrorInvalidValue;
    }
    const int mi = static_cast<int>(m);
    using H = _Float16;
    if (x_f16 && y_f16) return dispatch_tokens<H, H>(w, x, y, mi, n, k, stream);
    if (x_f16) return dispatch_tokens<H, float>(w, x, y, mi, n, k, stream);
    if (y_f16) return dispatch_tokens<float, H>(w, x, y, mi, n, k, stream);
    return dispatch_tokens<float, float>(w, x, y, mi, n, k, stream);
}

hipError_t launch_q8_0_gemv(const uint8_t *w, const float *x, const float *r, float *y, int64_t n, int64_t k,
                            hipStream_t stream) {
    if (n == 0) return hipSuccess;
    if (k == 0) return r != nullptr ? launch_copy(y, r, n, stream) : launch_fill_zero(y, n, stream);
    const GemvJob job{w, y, r, n};
    // the streaming kernels need dword-aligned groups: an even number of
    // blocks per row and a 4-byte aligned matrix
    if (k % 64 != 0 || (reinterpret_cast<uintptr_t>(w) & 3) != 0) {
        return launch_generic<Q8_0Format, float, float, false>(w, nullptr, x, r, y, n, k, stream);
    }
    if (Q4K_Q8_0_STAGE && k % 256 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0) {
        if (k <= 4096) return dispatch_short<Q8_0StagedFormat, float, float, false>(&job, 1, nullptr, x, k, stream);
        // rows of 129-192 groups: the three-slice split kernel, whose ring
        // (one 4352-byte slice per wave, 12 waves) fits in LDS beside the
        // activations
        if (k > 8192 && k <= 12288)
            return launch_split<Q8_0StagedFormat, float, float, 3, 4, false, 1 + Q4K_SPLIT3_SLOTS, 3>(w, nullptr, x, r,
                                                                                                     y, n, k, stream);
    }
    return dispatch<Q8_0Format, float, float, false>(&job, 1, nullptr, x, k, stream);
}

}  // namespace q4k
