// Read-only streaming kernel: the achievable HBM read rate on this device,
// reported beside the GEMV measurements for context (the roofline stays the
// published peak).  Not part of the q4k C ABI: a separate library used by
// the benchmark only.
//
// Every 16-byte chunk of the buffer is read exactly once.  Thread t of a
// grid of T threads reads chunks t, t + T, t + 2T, ... with UNROLL loads in
// flight, so a wave reads 1 KB of consecutive bytes per load and the whole
// grid sweeps the buffer front to back.  The loaded words are folded with
// XOR into one word per thread, written to `out`, so that no load is dead.
// AUX is the loads' cache policy: 0 the default, 2 non-temporal (every line
// is read whole by one load, where the non-temporal policy streams faster).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int UNROLL, int AUX>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t *__restrict__ p, int64_t chunks,
                                                          uint32_t *__restrict__ out) {
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nth = static_cast<int64_t>(gridDim.x) * 256;
    // chunks < 2^27 (the host checks): every byte offset fits the 32-bit
    // offset of a buffer load, and offsets past the end read zeros
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p), 0, static_cast<int>(chunks * 16), 0x00020000);
    uint32_t acc = 0;
    for (int64_t base = tid; base < chunks; base += nth * UNROLL) {
        u32x4_t v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t c = base + u * nth;
            const uint32_t off = c < chunks ? static_cast<uint32_t>(c * 16) : 0x80000000u;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, AUX);
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    out[tid] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, at most 2 GiB - 16) at device pointer p
// once on `stream` with `grid` workgroups of 256 threads, `unroll` (4 or 8)
// loads in flight per thread and cache policy `policy` (0 default, 2
// non-temporal); out: device buffer of grid * 256 words.  Returns a
// hipError_t value (0: launched).
extern "C" __attribute__((visibility("default"))) int q4k_stream_read(const void *p, int64_t bytes, void *out,
                                                                      int grid, int unroll, int policy,
                                                                      void *stream) {
    if (p == nullptr || out == nullptr || bytes <= 0 || bytes % 16 != 0 || bytes >= (int64_t{1} << 31) ||
        grid <= 0 || (unroll != 4 && unroll != 8) || (policy != 0 && policy != 2)) {
        return static_cast<int>(hipErrorInvalidValue);
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const auto *src = static_cast<const uint8_t *>(p);
    auto *dst = static_cast<uint32_t *>(out);
    const int64_t chunks = bytes / 16;
    if (unroll == 4 && policy == 0) hipLaunchKernelGGL((stream_read_kernel<4, 0>), dim3(grid), dim3(256), 0, s, src, chunks, dst);
    else if (unroll == 4) hipLaunchKernelGGL((stream_read_kernel<4, 2>), dim3(grid), dim3(256), 0, s, src, chunks, dst);
    else if (policy == 0) hipLaunchKernelGGL((stream_read_kernel<8, 0>), dim3(grid), dim3(256), 0, s, src, chunks, dst);
    else hipLaunchKernelGGL((stream_read_kernel<8, 2>), dim3(grid), dim3(256), 0, s, src, chunks, dst);
    return static_cast<int>(hipGetLastError());
}
