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

// Weight loads that go straight to LDS (no registers): lane l's 16 bytes at
// descriptor offset voff land at dst + 16 l, dst being wave-uniform (it goes
// to M0).  Such loads read whole lines in one instruction, so they take the
// non-temporal policy, which streams faster than the default one when every
// line is consumed by a single load (and slower when several loads share a
// line, as the register loads above do).
#ifndef Q4K_STAGE_CPOL
#define Q4K_STAGE_CPOL 2
#endif

__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0,
                                             Q4K_STAGE_CPOL);
}

// The same with 4 bytes per lane (256 bytes per wave).
__device__ __forceinline__ void buffer_load4_lds(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 4, voff, 0, 0,
                                             Q4K_STAGE_CPOL);
}

// BYTES (a multiple of 256) contiguous bytes from descriptor offset 0 to LDS
// at dst (wave-uniform): whole kilobytes by 16-byte loads, the rest by 4-byte
// loads.  stage_loads<BYTES> is the number of load instructions, for wait_vm.
template <int BYTES>
constexpr int stage_loads() {
    return BYTES / 1024 + (BYTES % 1024) / 256;
}

template <int BYTES>
__device__ __forceinline__ void stage_bytes(__amdgpu_buffer_rsrc_t r, uint8_t *dst, int lane) {
    static_assert(BYTES % 256 == 0, "whole 256-byte pieces");
    constexpr int kFull = BYTES / 1024;
    constexpr int kTail = (BYTES % 1024) / 256;
#pragma unroll
    for (int i = 0; i < kFull; ++i) buffer_load16_lds(r, dst + i * 1024, i * 1024u + static_cast<uint32_t>(lane) * 16u);
#pragma unroll
    for (int i = 0; i < kTail; ++i)
        buffer_load4_lds(r, dst + kFull * 1024 + i * 256, kFull * 1024u + i * 256u + static_cast<uint32_t>(lane) * 4u);
}

// Waits for this wave's LDS reads (and scalar loads), nothing else; the empty
// asm statements keep the compiler from moving memory operations across it.
__device__ __forceinline__ void wait_lds_reads() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
    asm volatile("" ::: "memory");
}

// Waits until at most N vector memory operations of this wave are in flight.
// Loads complete in issue order, so this waits for everything issued before
// the last N operations.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is six bits");
    asm volatile("" ::: "memory");
    // vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// The 32-bit LDS byte address of a pointer into LDS.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

// Three 16-byte LDS reads, at LDS byte addresses a, b and b + 16 (each a
// multiple of 16), complete on return.  Written as one asm statement with its
// own lgkmcnt wait: the compiler then sees no LDS read and adds no wait for
// the staged weight loads still in flight to other slots (it cannot tell
// them apart and would wait for all of them); the caller waits for the
// slot's own loads (wait_vm).
__device__ __forceinline__ void lds_read_3x16(uint32_t a, uint32_t b, uint4 &ra, uint4 &rb, uint4 &rc) {
    u32x4_t x, y, z;
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %4\n\t"
        "ds_read_b128 %2, %4 offset:16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x), "=&v"(y), "=&v"(z)
        : "v"(a), "v"(b)
        : "memory");
    ra = make_uint4(x.x, x.y, x.z, x.w);
    rb = make_uint4(y.x, y.y, y.z, y.w);
    rc = make_uint4(z.x, z.y, z.z, z.w);
}

// One 16-byte LDS read at LDS byte address a (a multiple of 16), complete on
// return (see lds_read_3x16).
__device__ __forceinline__ uint4 lds_read_16(uint32_t a) {
    u32x4_t x;
    asm volatile(
        "ds_read_b128 %0, %1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x)
        : "v"(a)
        : "memory");
    return make_uint4(x.x, x.y, x.z, x.w);
}

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// operations complete, then s_barrier.  Unlike __syncthreads() it does not
// wait for loads still in flight to LDS (a workgroup release fence waits for
// those), so the weight stream keeps running across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

// The sums over the whole wave of two values at once, each the same bits as
// lane_group_sum<64> of it: one permlane32 swap of a and b leaves lanes 0-31
// with a's lane pairs (i, i+32) and lanes 32-63 with b's, added in the order
// swap32_sum adds them; the rest of the reduction then runs once for both
// halves, and a last swap hands every lane both totals.
__device__ __forceinline__ void wave_sum_pair(float &a, float &b) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    const unsigned r0 = s[0];
    const unsigned r1 = opaque_copy(s[1]);
    float v = __uint_as_float(r0) + __uint_as_float(r1);
    v = swap16_sum(v);
    v = dpp_add<0xb1>(v);
    v = dpp_add<0x4e>(v);
    v = dpp_add<0x141>(v);
    v = dpp_add<0x140>(v);
    const unsigned u = __float_as_uint(v);
    const auto t = __builtin_amdgcn_permlane32_swap(u, opaque_copy(u), false, false);
    a = __uint_as_float(t[0]);              // lanes 0-31 of v everywhere: a's sum
    b = __uint_as_float(opaque_copy(t[1]));  // lanes 32-63 of v everywhere: b's sum
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

// ---- a lower bound on a group's magnitude without its four largest values
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// (t1, t2) becomes the two largest of (t1, t2) and (u1, u2), both descending.
__device__ __forceinline__ void merge_top2(float &t1, float &t2, float u1, float u2) {
    const float n2 = fmaxf(fminf(t1, u1), fmaxf(t2, u2));
    t1 = fmaxf(t1, u1);
    t2 = n2;
}

template <int CTRL>
__device__ __forceinline__ void merge_top2_dpp(float &t1, float &t2) {
    merge_top2(t1, t2, dpp_mov<CTRL>(t1), dpp_mov<CTRL>(t2));
}

// For the non-negative values v (4 per lane) of an aligned group of W lanes
// (W = 16 or 32): a quick lower bound on the sum of the group's values other
// than its four largest, formed from non-negative terms only.  T is the
// second largest, over the lanes, of each lane's second largest value: two
// lanes hold two values >= T each, so the group's four largest are all >= T,
// and the sum of the values below T leaves them all out (with up to 4 + W - 2
// values in all, so it can fall well below the sum without the four largest;
// lane_group_rest_bound then gives that sum).
template <int W>
__device__ __forceinline__ float lane_group_rest_bound_quick(const float (&v)[4]) {
    static_assert(W == 16 || W == 32, "group width");
    const float p = fmaxf(v[0], v[1]), q = fminf(v[0], v[1]);
    const float r = fmaxf(v[2], v[3]), s = fminf(v[2], v[3]);
    float t1 = fmaxf(fminf(p, r), fmaxf(q, s));  // the lane's second largest
    float t2 = 0.0f;
    merge_top2_dpp<0xb1>(t1, t2);   // quad_perm [1,0,3,2]
    merge_top2_dpp<0x4e>(t1, t2);   // quad_perm [2,3,0,1]
    merge_top2_dpp<0x141>(t1, t2);  // row_half_mirror
    merge_top2_dpp<0x140>(t1, t2);  // row_mirror
    if constexpr (W == 32) merge_top2(t1, t2, __shfl_xor(t1, 16, kWave), __shfl_xor(t2, 16, kWave));
    float below = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) below += v[b] < t2 ? v[b] : 0.0f;
    if constexpr (W == 16) return lane_group_sum<16>(below);
    else return lane_group_sum<32>(below);
}

// (a, b) becomes (max, min).
__device__ __forceinline__ void order2(float &a, float &b) {
    const float hi = fmaxf(a, b);
    b = fminf(a, b);
    a = hi;
}

// t becomes the four largest of t and u, both descending.  The maxima of
// t[i] and u[3-i] are those four (a multiset), falling then rising; two
// rounds of compare-exchange (a bitonic merge) sort them.
__device__ __forceinline__ void merge_top4(float (&t)[4], const float (&u)[4]) {
    float c0 = fmaxf(t[0], u[3]), c1 = fmaxf(t[1], u[2]), c2 = fmaxf(t[2], u[1]), c3 = fmaxf(t[3], u[0]);
    order2(c0, c2);
    order2(c1, c3);
    order2(c0, c1);
    order2(c2, c3);
    t[0] = c0;
    t[1] = c1;
    t[2] = c2;
    t[3] = c3;
}

template <int CTRL>
__device__ __forceinline__ void merge_top4_dpp(float (&t)[4]) {
    const float u[4] = {dpp_mov<CTRL>(t[0]), dpp_mov<CTRL>(t[1]), dpp_mov<CTRL>(t[2]), dpp_mov<CTRL>(t[3])};
    merge_top4(t, u);
}

// For the non-negative values v (4 per lane) of an aligned group of W lanes
// (W = 16 or 32): a lower bound on the sum of the group's values other than
// its four largest, formed from non-negative terms only (no cancellation,
// whatever the spread).  Every lane's four values are sorted, then merged
// with its partner's into the four largest of both, over the lane pairings
// of lane_group_sum (after each step both partners hold the same four, so the
// next step merges disjoint sets); every lane ends with the group's four
// largest.  The values below the fourth largest, T, leave out the four
// largest (and any value tied with T), so their sum is the bound; it equals
// the sum without the four largest when no other value equals T.
template <int W>
__device__ __forceinline__ float lane_group_rest_bound(const float (&v)[4]) {
    static_assert(W == 16 || W == 32, "group width");
    float t[4] = {v[0], v[1], v[2], v[3]};
    order2(t[0], t[1]);
    order2(t[2], t[3]);
    order2(t[0], t[2]);
    order2(t[1], t[3]);
    order2(t[1], t[2]);
    merge_top4_dpp<0xb1>(t);   // quad_perm [1,0,3,2]
    merge_top4_dpp<0x4e>(t);   // quad_perm [2,3,0,1]
    merge_top4_dpp<0x141>(t);  // row_half_mirror
    merge_top4_dpp<0x140>(t);  // row_mirror
    if constexpr (W == 32) {
        const float u[4] = {__shfl_xor(t[0], 16, kWave), __shfl_xor(t[1], 16, kWave), __shfl_xor(t[2], 16, kWave),
                            __shfl_xor(t[3], 16, kWave)};
        merge_top4(t, u);
    }
    float below = 0.0f;
#pragma unroll
    for (int b = 0; b < 4; ++b) below += v[b] < t[3] ? v[b] : 0.0f;
    if constexpr (W == 16) return lane_group_sum<16>(below);
    else return lane_group_sum<32>(below);
}

// A lower bound on the magnitude of a group (W lanes, four values each)
// without its four largest, as tight as the test needs: `first` (the sum
// minus four times the largest) where it is at least `need`, else the quick
// bound where that is, else the exact one.  Each tier runs only in waves that
// hold a group the previous one did not clear; a group's lanes agree on every
// test, so the lane exchanges inside each bound stay within active groups.
template <int W>
__device__ __forceinline__ float rest_bound_tiers(const float (&mag)[4], float first, float need) {
    float rest = first;
    if (__builtin_amdgcn_ballot_w64(need > rest) != 0) {
        if (need > rest) rest = lane_group_rest_bound_quick<W>(mag);
        if (__builtin_amdgcn_ballot_w64(need > rest) != 0) {
            if (need > rest) rest = lane_group_rest_bound<W>(mag);
        }
    }
    return rest;
}

}  // namespace q4k
