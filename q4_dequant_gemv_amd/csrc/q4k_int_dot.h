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
#pragma once

#include <float.h>
#include <math.h>

#include "q4k_device.h"

namespace q4k {

// Activations of one 64-weight group, ready for the integer dot products.
struct XGroup {
    uint32_t limb[2][3][8];  // [sub-block of the pair][limb][dword], 4 signed bytes per dword
    int32_t sx[2];           // sum of X over each 32-weight sub-block
    float scale;             // x ~= X * scale (power of two); 0 if all x are 0; NaN if any is not finite
    uint32_t pad;
};
static_assert(sizeof(XGroup) == 208, "XGroup layout");

// Converts x[0 .. 64*ngroups) into XGroups, 16 threads per group, 4
// activations per thread.  BLOCK is a multiple of 64, so the 16 threads of a
// group are 16 aligned lanes of one wave and are either all active or all not.
// The activations are loaded first (load_x) so that a kernel can issue them
// ahead of its weight loads: waits are counted in issue order, so waiting for
// the activations then leaves the weight loads in flight.  NCH covers
// ngroups*16 <= NCH*BLOCK.
template <int NCH>
struct XLoaded {
    float v[NCH][4];
};

// T is float or _Float16 (f16 activations are widened exactly).
template <int BLOCK, int NCH, typename T>
__device__ __forceinline__ XLoaded<NCH> load_x(const T *x, int ngroups) {
    XLoaded<NCH> f;
    const int total = ngroups * 16;
    // every load is issued (items past the end re-read item 0) so that no
    // load sits in a branch; the unused values are dropped afterwards
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int it = static_cast<int>(threadIdx.x) + c * BLOCK;
        const T *p = x + 4 * (it < total ? it : 0);
#pragma unroll
        for (int b = 0; b < 4; ++b) f.v[c][b] = static_cast<float>(p[b]);
    }
    return f;
}

template <int BLOCK, int NCH>
__device__ __forceinline__ void prepare_x(const XLoaded<NCH> &f, int ngroups, XGroup *__restrict__ xg) {
    const int total = ngroups * 16;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int it = static_cast<int>(threadIdx.x) + c * BLOCK;
        if (it >= total) break;
        const int j = it >> 4;
        const int half = (it >> 3) & 1;
        const int i = it & 7;
        float v[4];
        float amax = 0.0f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            v[b] = f.v[c][b];
            float a = fabsf(v[b]);
            a = (a <= FLT_MAX) ? a : INFINITY;  // NaN counts as non-finite
            amax = fmaxf(amax, a);
        }
        amax = lane_group_max<16>(amax);  // DPP inside the 16-lane row: no LDS round trip
        const bool finite = amax <= FLT_MAX;
        const bool zero = amax == 0.0f;
        int sexp = 0;
        float scale = 0.0f;
        if (!finite) {
            scale = NAN;
        } else if (!zero) {
            const int e = ilogbf(amax);
            sexp = 21 - e;
            scale = ldexpf(1.0f, e - 21);
        }
        // Balanced digits by a bias: with X = X2*2^16 + X1*2^8 + X0 and every
        // Xj in [-128, 127], byte j of B = X + 0x808080 is Xj + 128 (B stays
        // below 2^24), so gathering byte j of the four values into one dword
        // (two rounds of byte permutes) and flipping each byte's top bit
        // gives the four Xj as signed bytes.
        uint32_t bx[4];
        int s = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int X = (finite && !zero) ? static_cast<int>(rintf(ldexpf(v[b], sexp))) : 0;
            s += X;
            bx[b] = static_cast<uint32_t>(X + 0x808080);
        }
        // v_perm_b32: byte i of the result is byte sel_i of {first (bytes 4-7), second (bytes 0-3)}
        const uint32_t t01 = __builtin_amdgcn_perm(bx[1], bx[0], 0x05010400u);  // bytes 0 and 1 of values 0, 1
        const uint32_t t23 = __builtin_amdgcn_perm(bx[3], bx[2], 0x05010400u);
        const uint32_t u01 = __builtin_amdgcn_perm(bx[1], bx[0], 0x07030602u);  // bytes 2 and 3 of values 0, 1
        const uint32_t u23 = __builtin_amdgcn_perm(bx[3], bx[2], 0x07030602u);
        const uint32_t l0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u) ^ 0x80808080u;
        const uint32_t l1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u) ^ 0x80808080u;
        const uint32_t l2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u) ^ 0x80808080u;
        s = lane_group_sum_int<8>(s);
        xg[j].limb[half][0][i] = l0;
        xg[j].limb[half][1][i] = l1;
        xg[j].limb[half][2][i] = l2;
        if (i == 0) xg[j].sx[half] = s;
        if ((it & 15) == 0) xg[j].scale = scale;
    }
}

// The general form for any number of groups (loads inside the loop).
template <int BLOCK>
__device__ __forceinline__ void prepare_x(const float *__restrict__ x, int ngroups, XGroup *__restrict__ xg) {
    const int total = ngroups * 16;
    for (int base = 0; base < total; base += BLOCK) {
        const XLoaded<1> f = load_x<BLOCK, 1, float>(x + 4 * base, (total - base + 15) / 16);
        prepare_x<BLOCK, 1>(f, (total - base + 15) / 16, xg + base / 16);
    }
}

// Per-lane register copy of one XGroup.
struct XRegs {
    uint32_t limb[2][3][8];
    int32_t sx[2];
    float scale;
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
template <typename XS>
__device__ __forceinline__ float group_dot(const GroupCodes &c, const XS &xs) {
    // The code and min products are rounded separately (no FMA), so a
    // sub-block whose weights all cancel (d*sc*q == dmin*m) gives exactly 0.
#pragma clang fp contract(off)
    int a00 = 0, a01 = 0, a02 = 0, a10 = 0, a11 = 0, a12 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
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

}  // namespace q4k
