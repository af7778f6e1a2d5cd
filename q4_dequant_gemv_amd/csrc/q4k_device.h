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

}  // namespace q4k
