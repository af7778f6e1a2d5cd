// q4k_dequant: Q4_K matrix -> dense f32, bit-exact.
//
// This is the "dequantize once to dense f32" step named under "Honest limits"
// in the qualia_core_db cuda_lane module docs, done on the GPU.  Each weight is
// f32(f32(d*sc)*q - f32(dmin*m)) with three separately rounded operations.
// (d*sc has at most 17 significant bits and dl*q at most 21, so both products
// are exact in f32 and only the subtraction rounds; FMA contraction is still
// switched off so the statement holds by construction.)
//
// Work split: one thread writes four consecutive outputs with one 16-byte
// store, so every store instruction of a wave covers 1 KiB of contiguous
// output; the operation is bound by those writes (4 bytes out per 0.5625 in).
// Large outputs use non-temporal stores (launch_dequant).
// A thread reads its super-block's 16-byte header and the one code dword
// holding its four nibbles; neighbouring threads re-read the same lines from
// cache.
#include "launch.h"
#include "q4k_device.h"

namespace q4k {

// NT: non-temporal stores (outputs larger than the Infinity Cache stream
// straight out instead of displacing it; see launch_dequant).
template <bool NT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ w, float *__restrict__ out,
                                                      int64_t total_quads) {
#pragma clang fp contract(off)
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total_quads; t += stride) {
        // quad t covers weights 4t..4t+3 of the flattened [n, k] matrix; since
        // k % 256 == 0, super-block index and row layout coincide:
        // super-block t/64 holds them, at in-block position e0 = 4*(t % 64).
        const int64_t blk = t >> 6;
        const int e0 = static_cast<int>(t & 63) * 4;
        const uint8_t *b = w + blk * kBlockBytes;
        const uint4 hdr = *reinterpret_cast<const uint4 *>(b);
        const int g = e0 >> 6;          // 64-weight group
        const int r = e0 & 63;          // position inside the group
        const int j = 2 * g + (r >> 5); // sub-block
        const int l = r & 31;           // code byte inside the group
        const uint32_t codes = *reinterpret_cast<const uint32_t *>(b + 16 + 32 * g + l);
        const uint32_t nib = (r < 32) ? (codes & 0x0f0f0f0fu) : ((codes >> 4) & 0x0f0f0f0fu);
        int sc, m;
        scale_min(hdr.y, hdr.z, hdr.w, j, sc, m);
        const float d = half_bits_to_float(hdr.x);
        const float dmin = half_bits_to_float(hdr.x >> 16);
        const float dl = d * static_cast<float>(sc);
        const float ml = dmin * static_cast<float>(m);
        float4 o;
        o.x = dl * static_cast<float>(nib & 0xffu) - ml;
        o.y = dl * static_cast<float>((nib >> 8) & 0xffu) - ml;
        o.z = dl * static_cast<float>((nib >> 16) & 0xffu) - ml;
        o.w = dl * static_cast<float>(nib >> 24) - ml;
        if constexpr (NT) {
            __builtin_nontemporal_store(o.x, out + 4 * t);
            __builtin_nontemporal_store(o.y, out + 4 * t + 1);
            __builtin_nontemporal_store(o.z, out + 4 * t + 2);
            __builtin_nontemporal_store(o.w, out + 4 * t + 3);
        } else {
            *reinterpret_cast<float4 *>(out + 4 * t) = o;
        }
    }
}

hipError_t launch_dequant(const uint8_t *w, float *out, int64_t n, int64_t k, hipStream_t stream) {
    const int64_t total_quads = n * (k / 4);
    if (total_quads == 0) return hipSuccess;
    const int threads = 256;
    const int64_t want = (total_quads + threads - 1) / threads;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 32;
    const int grid = static_cast<int>(want < cap ? want : cap);
    // Outputs of 256 MiB or more (beyond the device's 256 MB Infinity Cache)
    // are written with non-temporal stores: the 0.8B lm_head (1 GB of f32)
    // went from 3.80 to 5.30 TB/s of reads and writes; a 201 MB output (the 9B
    // gate), which the cache holds, is 2 % faster with ordinary stores.
    if (total_quads * 16 >= (int64_t{256} << 20)) {
        hipLaunchKernelGGL(dequant_kernel<true>, dim3(grid), dim3(threads), 0, stream, w, out, total_quads);
    } else {
        hipLaunchKernelGGL(dequant_kernel<false>, dim3(grid), dim3(threads), 0, stream, w, out, total_quads);
    }
    return hipGetLastError();
}

}  // namespace q4k
