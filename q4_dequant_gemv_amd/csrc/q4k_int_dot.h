// Integer dot products of Q4_K codes with activations on the vector ALUs
// (v_dot4_i32_i8), shared by the batch-1 GEMV, the SwiGLU GEMV and the
// few-token form of the batched call (the same kernels with token tiles).
//
// A 64-weight group is one sub-block pair (2g, 2g+1) of a super-block: its 32
// code bytes hold the 32 weights of sub-block 2g in their low nibbles and the
// 32 weights of sub-block 2g+1 in their high nibbles, at matching positions.
//
// Activations of a group are converted once to integers
//     X = rint(x * 2^(21-e)),   2^e <= max|x| < 2^(e+1),   |X| <= 2^22,
// so x = X * 2^(e-21) to within 2^-22 of the group's largest magnitude, and
// X = X2*2^16 + X1*2^8 + X0 with X0, X1 in [-128, 127] and |X2| <= 64 (each
// limb a signed byte).  For a sub-block of 32 codes (q <= 15) the limb sums
// stay within 32*15*128 = 61440 (|X2| sums within 30720), so the recombined
// S = sum q*X is below 30720*2^16 + 61440*2^8 + 61440 < 2^31: all integer
// arithmetic is exact.
//
// That representation is accurate relative to the group's largest |x|, not
// to each activation: every activation is rounded to a step of 2^(e-21).  A
// few outliers far above the rest of their group would make that step coarse
// for all the others, and an outlier's weight may be zero.  prepare_x
// therefore compares, per group, the total rounding E = sum_k |x_k - X_k
// 2^(e-21)| with S4, the sum of the group's |x| other than its four largest
// (what is left of sum |w x| if the weights of up to four outliers are zero),
// through a lower bound formed without cancellation (quad_rest_bound).  A
// group with E > 2^-15 times that bound is flagged, and a wave that meets a
// flagged group multiplies every weight in f32 instead (exact_group_dot): the weight is
// dequantized as the dequant kernel does and each product w * x is rounded
// once, so every activation keeps its full precision.  On the integer path a
// group's rounding therefore adds at most 2^-15 * max_k |w_k| * S4 to a row's
// result (S4 is at least the bound).  Both sums are formed from terms exact
// in f32 (their own rounding is a few 2^-24).
#pragma once

#include <type_traits>

#include <float.h>
#include <math.h>

#include "q4k_device.h"

namespace q4k {

// Activations of one 64-weight group, ready for the integer dot products.
struct XGroup {
    uint32_t limb[2][3][8];  // [sub-block of the pair][limb][dword], 4 signed bytes per dword
    int32_t sx[2];           // sum of X over each 32-weight sub-block
    float scale;             // x ~= X * scale (power of two); 0 if all x are 0; NaN if any is not finite
    uint32_t inexact;        // 1: the group needs the f32 path (rounding above 2^-15 of its magnitude bar the top 4)
};
static_assert(sizeof(XGroup) == 208, "XGroup layout");

// Converts x[0 .. 64*ngroups) into XGroups, 4 threads per group, 16
// consecutive activations per thread (an item: item it holds activations
// 16*it .. 16*it+15, the quarter it & 3 of group it >> 2).  BLOCK is a
// multiple of 64, so the 4 threads of a group are 4 aligned lanes (a quad) of
// one wave and are either all active or all not.  The activations are loaded
// first (load_x) so that a kernel can issue them ahead of its weight loads:
// waits are counted in issue order, so waiting for the activations then
// leaves the weight loads in flight.  NCH covers ngroups*4 <= NCH*BLOCK
// (x_chunks).
constexpr int kXItem = 16;  // activations per thread and chunk

constexpr int x_chunks(int max_groups, int block) { return (max_groups * 4 + block - 1) / block; }

template <int NCH>
struct XLoaded {
    float v[NCH][kXItem];
};

// T is float or _Float16 (f16 activations are widened exactly).
// COHERENT: device-coherent loads (agent scope), for activations that other
// workgroups of the same launch wrote with device-coherent stores.
template <int BLOCK, int NCH, typename T, bool COHERENT = false>
__device__ __forceinline__ XLoaded<NCH> load_x(const T *x, int ngroups) {
    static_assert(!COHERENT || std::is_same_v<T, float>, "coherent loads of f32 activations");
    XLoaded<NCH> f;
    const int total = ngroups * 4;
    // every load is issued (items past the end re-read item 0) so that no
    // load sits in a branch; the unused values are dropped afterwards
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int it = static_cast<int>(threadIdx.x) + c * BLOCK;
        const T *p = x + kXItem * (it < total ? it : 0);
#pragma unroll
        for (int b = 0; b < kXItem; ++b) {
            if constexpr (COHERENT) {
                f.v[c][b] = __hip_atomic_load(p + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                f.v[c][b] = static_cast<float>(p[b]);
            }
        }
    }
    return f;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Maximum over the quads of unsigned values (DPP, no LDS).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    return umax(static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, true)), v);
}

// For the 64 non-negative values of a group (16 per lane of a quad): a lower
// bound on the sum of the values other than the four largest, formed from
// non-negative terms only (no cancellation, whatever the spread).  Each lane
// keeps the four largest of its values (sorted runs of four, merged), the
// quad's lanes merge theirs over the lane pairings of lane_group_sum (after
// each step both partners hold the same four, so the next step merges
// disjoint sets), and every lane ends with the group's four largest.  The
// values below the fourth largest, T, leave out the four largest (and any
// value tied with T), so their sum is the bound; it equals the sum without
// the four largest when no other value equals T.
__device__ __forceinline__ float quad_rest_bound(const float (&v)[kXItem]) {
    float t[4];
#pragma unroll
    for (int r = 0; r < kXItem / 4; ++r) {
        float u[4] = {v[4 * r], v[4 * r + 1], v[4 * r + 2], v[4 * r + 3]};
        order2(u[0], u[1]);
        order2(u[2], u[3]);
        order2(u[0], u[2]);
        order2(u[1], u[3]);
        order2(u[1], u[2]);
        if (r == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) t[i] = u[i];
        } else {
            merge_top4(t, u);
        }
    }
    merge_top4_dpp<0xb1>(t);  // quad_perm [1,0,3,2]
    merge_top4_dpp<0x4e>(t);  // quad_perm [2,3,0,1]
    float below = 0.0f;
#pragma unroll
    for (int b = 0; b < kXItem; ++b) below += v[b] < t[3] ? v[b] : 0.0f;
    return lane_group_sum<4>(below);
}

// Converts the loaded activations to XGroups.  A group's `inexact` is 1 if
// its total rounding E exceeds 2^-15 of S4, its magnitude without its four
// largest (see above).  Non-finite groups are not flagged (their results are
// NaN on either path, whatever their integers).  Per chunk:
//  - the largest magnitude is taken on the bit patterns of |x| (for
//    non-negative floats integer order is numeric order, and every NaN
//    pattern lies above infinity's);
//  - X = rint(x * 2^(21-e)) comes from one addition of 1.5 * 2^23: the sum
//    lies in [2^23, 2^24], where the spacing of floats is 1, so it is rounded
//    to the nearest integer, ties to even, as rint does, and its bit pattern
//    is 0x4B400000 + X;
//  - the lower bound on S4 is first the sum of the magnitudes less four times
//    the largest (no sort).  E is at most 64 * 1/2 = 2^5 units of 2^(e-21), so
//    where that bound reaches 2^20 units the group passes whatever E is, and
//    only waves holding a group below it form E and, where E * 2^15 exceeds
//    the first bound, the exact one (quad_rest_bound).
template <int BLOCK, int NCH>
__device__ __forceinline__ void prepare_x(const XLoaded<NCH> &f, int ngroups, XGroup *__restrict__ xg) {
    const int total = ngroups * 4;
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int it = static_cast<int>(threadIdx.x) + c * BLOCK;
        if (it >= total) break;  // whole quads leave together
        uint32_t mb = 0;
#pragma unroll
        for (int b = 0; b < kXItem; ++b) mb = umax(mb, __float_as_uint(f.v[c][b]) & 0x7fffffffu);
        mb = dpp_max_u32<0xb1>(mb);
        mb = dpp_max_u32<0x4e>(mb);
        const bool finite = mb < 0x7f800000u;
        const bool zero = mb == 0u;
        const bool live = finite && !zero;
        const float amax = __uint_as_float(mb);
        const int e = __builtin_amdgcn_frexp_expf(amax) - 1;  // ilogb of a finite non-zero amax
        const int sexp = live ? 21 - e : 0;
        const float scale = !finite ? NAN : (zero ? 0.0f : ldexpf(1.0f, e - 21));
        const float amax_s = live ? ldexpf(amax, sexp) : 0.0f;
        // v * 2^sexp is exact in f32 (a group that is not live keeps its
        // values: zeros give X = 0, and a non-finite group's integers are
        // never used, its scale being NaN)
        float sv[kXItem];
        uint32_t bx[kXItem];
#pragma unroll
        for (int b = 0; b < kXItem; ++b) {
            sv[b] = ldexpf(f.v[c][b], sexp);
            bx[b] = __float_as_uint(sv[b] + kMagic) - (0x4B400000u - 0x808080u);
        }
        float asum[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            asum[r] = (fabsf(sv[4 * r]) + fabsf(sv[4 * r + 1])) + (fabsf(sv[4 * r + 2]) + fabsf(sv[4 * r + 3]));
        }
        const float first = lane_group_sum<4>((asum[0] + asum[1]) + (asum[2] + asum[3])) - 4.0f * amax_s;
        uint32_t flag = 0u;
        const bool quick = !live || first >= 1048576.0f;
        if (__builtin_amdgcn_ballot_w64(!quick) != 0) {
            // rounding and magnitudes in units of 2^(e-21)
            float round_sum = 0.0f;
            float mag[kXItem];
#pragma unroll
            for (int b = 0; b < kXItem; ++b) {
                const float r = (sv[b] + kMagic) - kMagic;  // rint(sv), exactly
                round_sum += fabsf(sv[b] - r);
                mag[b] = fabsf(sv[b]);
            }
            const float need = lane_group_sum<4>(round_sum) * 32768.0f;
            float rest = first;
            if (__builtin_amdgcn_ballot_w64(live && need > rest) != 0) {
                const float exact = quad_rest_bound(mag);
                if (need > rest) rest = exact;
            }
            flag = live && need > rest ? 1u : 0u;
        }
        const int j = it >> 2;
        const int q = it & 3;
        const int half = q >> 1;
        // Balanced digits by a bias: with X = X2*2^16 + X1*2^8 + X0 and every
        // Xj in [-128, 127], byte j of B = X + 0x808080 is Xj + 128 (B stays
        // below 2^24), so gathering byte j of four values into one dword (two
        // rounds of byte permutes) and flipping each byte's top bit gives the
        // four Xj as signed bytes.
        // v_perm_b32: byte i of the result is byte sel_i of {first (bytes 4-7), second (bytes 0-3)}
        uint4 limb[3];
        uint32_t *l0 = &limb[0].x, *l1 = &limb[1].x, *l2 = &limb[2].x;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t *b4 = &bx[4 * d];
            const uint32_t t01 = __builtin_amdgcn_perm(b4[1], b4[0], 0x05010400u);  // bytes 0, 1 of values 0, 1
            const uint32_t t23 = __builtin_amdgcn_perm(b4[3], b4[2], 0x05010400u);
            const uint32_t u01 = __builtin_amdgcn_perm(b4[1], b4[0], 0x07030602u);  // bytes 2, 3 of values 0, 1
            const uint32_t u23 = __builtin_amdgcn_perm(b4[3], b4[2], 0x07030602u);
            l0[d] = __builtin_amdgcn_perm(t23, t01, 0x05040100u) ^ 0x80808080u;
            l1[d] = __builtin_amdgcn_perm(t23, t01, 0x07060302u) ^ 0x80808080u;
            l2[d] = __builtin_amdgcn_perm(u23, u01, 0x05040100u) ^ 0x80808080u;
        }
        // sum of the sixteen X (the biases removed; exact in 32-bit arithmetic),
        // then over the two lanes of the sub-block
        uint32_t bsum = 0u;
#pragma unroll
        for (int b = 0; b < kXItem; ++b) bsum += bx[b];
        bsum -= static_cast<uint32_t>(kXItem) * 0x808080u;
        const int s = dpp_add_int<0xb1>(static_cast<int>(bsum));
        uint4 *dst = reinterpret_cast<uint4 *>(&xg[j].limb[half][0][4 * (q & 1)]);
        dst[0] = limb[0];  // limb l of the half starts 8 dwords after limb l-1
        dst[2] = limb[1];
        dst[4] = limb[2];
        if ((q & 1) == 0) xg[j].sx[half] = s;
        if (q == 0) {
            xg[j].scale = scale;
            xg[j].inexact = flag;
        }
    }
}

// Per-lane register copy of one XGroup.
struct XRegs {
    uint32_t limb[2][3][8];
    int32_t sx[2];
    float scale;
    uint32_t inexact;
};

__device__ __forceinline__ void load_xregs(const XGroup &g, XRegs &r) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int l = 0; l < 3; ++l) {
#pragma unroll
            for (int i = 0; i < 8; ++i) r.limb[h][l][i] = g.limb[h][l][i];
        }
        r.sx[h] = g.sx[h];
    }
    r.scale = g.scale;
    r.inexact = g.inexact;
}

// The weights of one group, decoded: codes as bytes 0..15 (four per dword) for
// each sub-block of the pair, and the two sub-blocks' d*sc and dmin*m.
struct GroupCodes {
    uint32_t lo[8];  // sub-block 2g
    uint32_t hi[8];  // sub-block 2g+1
    float dl0, ml0, dl1, ml1;
};

__device__ __forceinline__ void decode_group(const uint4 &hdr, const uint4 &qa, const uint4 &qb,
                                             const PairSelect &ps, GroupCodes &c) {
    const float d = half_bits_to_float(hdr.x);
    const float dmin = half_bits_to_float(hdr.x >> 16);
    uint32_t scp, mp;
    scale_min_pair(hdr.y, hdr.z, hdr.w, ps, scp, mp);
    c.dl0 = d * static_cast<float>(scp & 0xffu);
    c.ml0 = dmin * static_cast<float>(mp & 0xffu);
    c.dl1 = d * static_cast<float>((scp >> 8) & 0xffu);
    c.ml1 = dmin * static_cast<float>((mp >> 8) & 0xffu);
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        c.lo[i] = q[i] & 0x0f0f0f0fu;
        c.hi[i] = (q[i] >> 4) & 0x0f0f0f0fu;
    }
}

// sum over the group of w*x, in units of the activation scale (multiply the
// result by the group's `scale`).  XS is XGroup (LDS) or XRegs (registers).
// v_dot4_i32_i8 with a zero accumulator (for the first product of a chain:
// the builtin with 0 becomes a move of 0 and the accumulate-in-place form)
__device__ __forceinline__ int sdot4_first(int a, int b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

template <typename XS>
__device__ __forceinline__ float group_dot(const GroupCodes &c, const XS &xs) {
    // The code and min products are rounded separately (no FMA), so a
    // sub-block whose weights all cancel (d*sc*q == dmin*m) gives exactly 0.
#pragma clang fp contract(off)
    const int lo0 = static_cast<int>(c.lo[0]);
    const int hi0 = static_cast<int>(c.hi[0]);
    int a00 = sdot4_first(lo0, static_cast<int>(xs.limb[0][0][0]));
    int a01 = sdot4_first(lo0, static_cast<int>(xs.limb[0][1][0]));
    int a02 = sdot4_first(lo0, static_cast<int>(xs.limb[0][2][0]));
    int a10 = sdot4_first(hi0, static_cast<int>(xs.limb[1][0][0]));
    int a11 = sdot4_first(hi0, static_cast<int>(xs.limb[1][1][0]));
    int a12 = sdot4_first(hi0, static_cast<int>(xs.limb[1][2][0]));
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        const int lo = static_cast<int>(c.lo[i]);
        const int hi = static_cast<int>(c.hi[i]);
        a00 = __builtin_amdgcn_sdot4(lo, static_cast<int>(xs.limb[0][0][i]), a00, false);
        a01 = __builtin_amdgcn_sdot4(lo, static_cast<int>(xs.limb[0][1][i]), a01, false);
        a02 = __builtin_amdgcn_sdot4(lo, static_cast<int>(xs.limb[0][2][i]), a02, false);
        a10 = __builtin_amdgcn_sdot4(hi, static_cast<int>(xs.limb[1][0][i]), a10, false);
        a11 = __builtin_amdgcn_sdot4(hi, static_cast<int>(xs.limb[1][1][i]), a11, false);
        a12 = __builtin_amdgcn_sdot4(hi, static_cast<int>(xs.limb[1][2][i]), a12, false);
    }
    const int s0 = a02 * 65536 + a01 * 256 + a00;
    const int s1 = a12 * 65536 + a11 * 256 + a10;
    const float t0 = c.dl0 * static_cast<float>(s0) - c.ml0 * static_cast<float>(xs.sx[0]);
    const float t1 = c.dl1 * static_cast<float>(s1) - c.ml1 * static_cast<float>(xs.sx[1]);
    return t0 + t1;
}

// A pointer the optimiser cannot follow, and that it takes to depend on
// a0 and a1: the f32 path reads its activations from memory for every row.
// Without this the loop-invariant loads would be hoisted out of the row loop,
// or all 64 issued at once, into 64 or more registers per token, which would
// raise the register budget of the whole kernel, integer path included.  No
// instruction is emitted.
// The result is a global-memory pointer (the activations are device memory),
// so its reads are global loads, counted on the vector-memory counter only.
template <typename T>
using global_ptr = const __attribute__((address_space(1))) T *;

template <typename T>
__device__ __forceinline__ global_ptr<T> opaque_after(const T *p, float a0, float a1) {
    uint64_t u = reinterpret_cast<uint64_t>(p);
    asm volatile("" : "+v"(u) : "v"(a0), "v"(a1));
    return (global_ptr<T>)u;
}

// A wave-uniform int the optimiser takes to depend on `after` (no
// instruction): orders a row's loads after the previous row's result.
__device__ __forceinline__ int opaque_int_after(int v, float after) {
    asm volatile("" : "+s"(v) : "v"(after));
    return v;
}

// sum over the group of w * x in f32 with every weight dequantized on its
// own, w = fma(d*sc, q, -dmin*m) (d*sc*q is exact in f32, so this is the
// correctly rounded weight the dequant kernel produces), and each product
// rounded once (FMA).  xs: the group's 64 activations in memory, float or
// _Float16 (weight 64g+l of the super-block pairs with xs[l] for the low
// nibbles, xs[32+l] for the high).  The activations are read a quarter at a
// time, each quarter's address depending on the sums so far (opaque_after),
// so at most 16 of them are in registers at once; the first quarter's
// address depends on `after` (a caller's previous result, to keep several
// rows' reads from being issued together, or a constant).
//
// A non-finite activation makes the result NaN, as on the integer path: the
// sum of 0 * x over the group (0 for finite x, NaN otherwise) is added.
template <typename T>
__device__ __forceinline__ float exact_group_dot(const GroupCodes &c, const T *xs, float after = 0.0f) {
    // each quarter's eight products per sub-block are summed on their own,
    // then added to the running sums: no chain of roundings is longer than 12
    float a0 = 0.0f, a1 = 0.0f, nf = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const global_ptr<T> p = opaque_after(xs, h == 0 ? after : a0, a1);
        float q0 = 0.0f, q1 = 0.0f;
#pragma unroll
        for (int i = 2 * h; i < 2 * h + 2; ++i) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float ql = static_cast<float>((c.lo[i] >> (8 * b)) & 0xffu);
                const float qh = static_cast<float>((c.hi[i] >> (8 * b)) & 0xffu);
                const float xl = static_cast<float>(p[4 * i + b]);
                const float xh = static_cast<float>(p[32 + 4 * i + b]);
                q0 = fmaf(fmaf(c.dl0, ql, -c.ml0), xl, q0);
                q1 = fmaf(fmaf(c.dl1, qh, -c.ml1), xh, q1);
                nf = fmaf(xl, 0.0f, fmaf(xh, 0.0f, nf));
            }
        }
        a0 += q0;
        a1 += q1;
    }
    return (a0 + a1) + nf;
}

}  // namespace q4k
