// Device-side building blocks shared by the Q4_K kernels (gfx950, wave64).
//
// Super-block layout (GGUF Q4_K; the pages' model files are Q4_K_M GGUF files,
// issue #3346): 144 bytes = d (f16) | dmin (f16) | 12 bytes of six-bit scales
// and mins | 128 code bytes.  Code byte 32g+l holds weight 64g+l (low nibble,
// sub-block 2g) and weight 64g+32+l (high nibble, sub-block 2g+1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

constexpr int kBlockBytes = 144;
constexpr int kBlockWeights = 256;
constexpr int kWave = 64;

// One 16-byte global load.  Weights are streamed once, so the load is marked
// non-temporal to keep the activations resident in L2.
__device__ __forceinline__ uint4 load_stream16(const uint8_t *p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Streaming loads through a buffer resource: the 128-bit descriptor (base,
// byte count) lives in scalar registers and each lane adds a 32-bit offset.
// Loads at or past `bytes` return zeros instead of touching memory, which
// covers ragged row tails without a branch around the loads.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const uint8_t *base, int bytes) {
    // dword 3 = 0x00020000: raw 32-bit data format, no swizzle, stride 0
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, bytes, 0x00020000);
}

// Cache policy bits of the weight loads (0: default; 2: non-temporal).
#ifndef Q4K_WEIGHT_CPOL
#define Q4K_WEIGHT_CPOL 0
#endif

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, Q4K_WEIGHT_CPOL);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, Q4K_WEIGHT_CPOL);
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// f16 bit patterns of 1024 + sc*q for the two codes of a nibble pair (the
// codes in the low and high 16 bits of `pair`, the scale in both halves of
// `sc2`): one packed 16-bit multiply-add, since sc*q <= 945 fits the 10-bit
// fraction of 1024.
__device__ __forceinline__ uint32_t pair_operand(uint32_t pair, uint32_t sc2) {
    const u16x2_t p = __builtin_bit_cast(u16x2_t, pair);
    const u16x2_t s = __builtin_bit_cast(u16x2_t, sc2);
    const u16x2_t magic = {0x6400, 0x6400};
    return __builtin_bit_cast(uint32_t, static_cast<u16x2_t>(p * s + magic));
}

// A value the caller knows is equal in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// IEEE binary16 (low 16 bits of `bits`) widened to f32; exact, denormals kept.
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits & 0xffffu)));
}

// Six-bit scale and min of sub-block j (0..7) from the 12 packed bytes, given
// as three little-endian dwords s0 (bytes 0-3), s1 (4-7), s2 (8-11).
// j < 4: scale = low six bits of byte j, min = low six bits of byte j+4.
// j >= 4 (i = j-4): low four bits from byte 8+i (scale: low nibble, min: high
// nibble), top two bits from the spare top bits of byte i (scale) and byte
// 4+i (min).
__device__ __forceinline__ void scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j, int &sc, int &m) {
    const int sh = 8 * (j & 3);
    const uint32_t b0 = (s0 >> sh) & 0xffu;
    const uint32_t b1 = (s1 >> sh) & 0xffu;
    const uint32_t b2 = (s2 >> sh) & 0xffu;
    if (j < 4) {
        sc = static_cast<int>(b0 & 63u);
        m = static_cast<int>(b1 & 63u);
    } else {
        sc = static_cast<int>((b2 & 15u) | ((b0 >> 6) << 4));
        m = static_cast<int>((b2 >> 4) | ((b1 >> 6) << 4));
    }
}

// The six-bit scales and mins of sub-blocks 2g and 2g+1 of one super-block,
// without branches: a lane-constant selector picks between the two packings
// (g < 2: low six bits of bytes 2g, 2g+1 of the first and second dword; g >= 2:
// low/high nibbles of bytes 2(g-2), 2(g-2)+1 of the third dword with the spare
// top two bits of the first/second dword above them).  Result: byte 0 holds
// sub-block 2g's value, byte 1 sub-block 2g+1's.
struct PairSelect {
    uint32_t sh;   // 16 * (g & 1): the two bytes of interest move to the bottom
    uint32_t s_hi; // 2 if g >= 2 else 0: top two bits into bit positions 4-5
    uint32_t s_lo; // 4 if g >= 2 else 0: min nibble (high) into the low nibble
    uint32_t m_lo; // 0x0f0f if g >= 2 else 0: keep the nibble part
    uint32_t m_hi; // 0x3030 if g >= 2 else 0x3f3f
};

__device__ __forceinline__ PairSelect pair_select(int g) {
    const bool hi = g >= 2;
    return PairSelect{16u * static_cast<uint32_t>(g & 1), hi ? 2u : 0u, hi ? 4u : 0u, hi ? 0x0f0fu : 0u,
                      hi ? 0x3030u : 0x3f3fu};
}

__device__ __forceinline__ void scale_min_pair(uint32_t s0, uint32_t s1, uint32_t s2, const PairSelect &ps,
                                               uint32_t &sc_pair, uint32_t &m_pair) {
    const uint32_t a = s0 >> ps.sh, b = s1 >> ps.sh, c = s2 >> ps.sh;
    sc_pair = (c & ps.m_lo) | ((a >> ps.s_hi) & ps.m_hi);
    m_pair = ((c >> ps.s_lo) & ps.m_lo) | ((b >> ps.s_hi) & ps.m_hi);
}

// Sum over aligned groups of W lanes (W a power of two, W <= 64); every lane of
// the group ends with the group's sum.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

template <int W>
__device__ __forceinline__ int group_sum_int(int v) {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float silu(float t) { return t / (1.0f + __expf(-t)); }

// ---- cross-lane sums on the VALU (no LDS): DPP inside 16-lane rows and the
// gfx950 permlane swaps across rows.  Every lane ends with its group's sum.
// (every control used here has a source lane for every lane, so bound_ctrl
// never applies; with it set the move folds into a single v_add_f32_dpp)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true);
    return __builtin_bit_cast(float, moved) + v;
}

// Sum over aligned groups of W lanes, W in {4, 8, 16, 32, 64}.
//  quad_perm [1,0,3,2] pairs lanes i, i^1; quad_perm [2,3,0,1] pairs i, i^2;
//  row_half_mirror pairs i, 7-i inside 8 lanes; row_mirror pairs i, 15-i
//  inside 16 (after the previous steps every lane of the smaller group holds
//  the same value, so mirrored partners complete the larger group).
//  permlane16_swap(v, v) returns (rows 0,0,2,2) and (rows 1,1,3,3): their sum
//  adds rows 2r and 2r+1; permlane32_swap(v, v) likewise adds the halves.
//  The swaps return two registers; hipcc 7.2 was seen to fold the float sum of
//  the pair into twice the first element.  Both the second operand and the
//  second result pass through an empty register-only asm statement, which
//  keeps them distinct values to the optimiser (no instruction is emitted).
__device__ __forceinline__ unsigned opaque_copy(unsigned v) {
    asm("" : "+v"(v));
    return v;
}

__device__ __forceinline__ float swap16_sum(float v) {
    const unsigned u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
    const unsigned r0 = s[0];
    const unsigned r1 = opaque_copy(s[1]);
    return __uint_as_float(r0) + __uint_as_float(r1);
}

__device__ __forceinline__ float swap32_sum(float v) {
    const unsigned u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
    const unsigned r0 = s[0];
    const unsigned r1 = opaque_copy(s[1]);
    return __uint_as_float(r0) + __uint_as_float(r1);
}

template <int W>
__device__ __forceinline__ float lane_group_sum(float v) {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32 || W == 64, "group width");
    if constexpr (W == 64) v = swap32_sum(v);
    if constexpr (W >= 32) v = swap16_sum(v);
    v = dpp_add<0xb1>(v);  // quad_perm [1,0,3,2]
    v = dpp_add<0x4e>(v);  // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v = dpp_add<0x141>(v);   // row_half_mirror
    if constexpr (W >= 16) v = dpp_add<0x140>(v);  // row_mirror
    return v;
}

// Integer sum over aligned groups of W lanes, W in {4, 8, 16} (inside one
// 16-lane row, so DPP alone reaches every partner).
template <int CTRL>
__device__ __forceinline__ int dpp_add_int(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true) + v;
}

template <int W>
__device__ __forceinline__ int lane_group_sum_int(int v) {
    static_assert(W == 4 || W == 8 || W == 16, "group width");
    v = dpp_add_int<0xb1>(v);
    v = dpp_add_int<0x4e>(v);
    if constexpr (W >= 8) v = dpp_add_int<0x141>(v);
    if constexpr (W >= 16) v = dpp_add_int<0x140>(v);
    return v;
}

// Maximum over aligned groups of W lanes (same lane pairings as lane_group_sum).
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true);
    return fmaxf(__builtin_bit_cast(float, moved), v);
}

__device__ __forceinline__ float swap16_max(float v) {
    const unsigned u = __float_as_uint(v);
    const auto s = __builtin_amdgcn_permlane16_swap(u, opaque_copy(u), false, false);
    const unsigned r0 = s[0];
    const unsigned r1 = opaque_copy(s[1]);
    return fmaxf(__uint_as_float(r0), __uint_as_float(r1));
}

template <int W>
__device__ __forceinline__ float lane_group_max(float v) {
    static_assert(W == 4 || W == 8 || W == 16 || W == 32, "group width");
    if constexpr (W >= 32) v = swap16_max(v);
    v = dpp_max<0xb1>(v);
    v = dpp_max<0x4e>(v);
    if constexpr (W >= 8) v = dpp_max<0x141>(v);
    if constexpr (W >= 16) v = dpp_max<0x140>(v);
    return v;
}

}  // namespace q4k
