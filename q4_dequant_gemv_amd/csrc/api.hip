// C ABI of libq4k.so (declared in include/q4k.h): host-side validation, then
// dispatch to the kernels on the caller's stream.  Validation follows the
// fail-before-dispatch practice of resolveMatmulOverride / failOrWarn in
// "@simulatte/doppler 0.1.7 -> 0.1.8" (matmul-selection.js): a bad argument is
// reported before anything is enqueued.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "q4k.h"
#include "launch.h"

namespace q4k {

namespace {

constexpr int kMaxDevices = 64;

__global__ void fill_zero_kernel(float *__restrict__ y, int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) y[i] = 0.0f;
}

__global__ void copy_kernel(float *y, const float *src, int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) y[i] = src[i];
}

__global__ void fill_zero_f16_kernel(_Float16 *y, int64_t count) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) {
        y[i] = static_cast<_Float16>(0.0f);
    }
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges, both non-empty).
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(b);
    if (na == 0 || nb == 0) return false;
    return pa < pb + nb && pb < pa + na;
}

// Largest element count accepted for any one tensor: keeps every byte offset
// inside int64 with room to spare.
constexpr int64_t kMaxElems = int64_t(1) << 56;

// Checks the sizes shared by every entry point and returns the weight bytes.
q4k_status check_shape(int64_t n, int64_t k, uint64_t *w_bytes) {
    if (n < 0 || k < 0) return Q4K_ERR_INVALID_ARG;
    if (k % Q4K_BLOCK_WEIGHTS != 0) return Q4K_ERR_UNSUPPORTED_SHAPE;
    if (k > 0 && n > kMaxElems / k) return Q4K_ERR_INVALID_ARG;
    *w_bytes = static_cast<uint64_t>(n) * static_cast<uint64_t>(k / Q4K_BLOCK_WEIGHTS) * Q4K_BLOCK_BYTES;
    return Q4K_OK;
}

q4k_status from_hip(hipError_t e) { return e == hipSuccess ? Q4K_OK : Q4K_ERR_LAUNCH; }

}  // namespace

int device_cu_count() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    const int64_t need = (count + 255) / 256;
    const int grid = static_cast<int>(need < 4096 ? need : 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, y, count);
    return hipGetLastError();
}

hipError_t launch_fill_zero_f16(_Float16 *y, int64_t count, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    const int64_t need = (count + 255) / 256;
    const int grid = static_cast<int>(need < 4096 ? need : 4096);
    hipLaunchKernelGGL(fill_zero_f16_kernel, dim3(grid), dim3(256), 0, stream, y, count);
    return hipGetLastError();
}

namespace {

// Scratch of the calls made without a workspace, kept per (device, stream)
// and reused: a call takes its stream's buffer (grown, stream-ordered, when it
// needs more), so back-to-back calls allocate nothing.  Calls on one stream
// run in order, and calls on different streams get different buffers, so no
// two calls in flight share one.  Buffers live until the process ends (at
// most kStreamScratchMax bytes per stream and kStreamScratchSlots streams);
// larger needs, a full table and calls recorded into a graph (whose
// allocations the graph must own) allocate and free per call as before.
constexpr int kStreamScratchSlots = 64;
constexpr int64_t kStreamScratchMax = int64_t{64} << 20;

struct StreamScratch {
    int dev;
    hipStream_t stream;
    uint8_t *ptr;
    int64_t bytes;
};

std::mutex g_stream_scratch_mutex;
StreamScratch g_stream_scratch[kStreamScratchSlots];
int g_stream_scratch_count = 0;

// *out = the stream's cached buffer of at least `total` bytes, or nullptr if
// the call should allocate for itself.
hipError_t stream_scratch(int64_t total, hipStream_t stream, uint8_t **out) {
    *out = nullptr;
    if (total > kStreamScratchMax) return hipSuccess;
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &status) != hipSuccess || status != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return hipSuccess;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_stream_scratch_mutex);
    StreamScratch *slot = nullptr;
    for (int i = 0; i < g_stream_scratch_count; ++i) {
        if (g_stream_scratch[i].dev == dev && g_stream_scratch[i].stream == stream) slot = &g_stream_scratch[i];
    }
    if (slot != nullptr && slot->bytes >= total) {
        *out = slot->ptr;
        return hipSuccess;
    }
    if (slot == nullptr) {
        if (g_stream_scratch_count == kStreamScratchSlots) return hipSuccess;
        slot = &g_stream_scratch[g_stream_scratch_count];
        *slot = StreamScratch{dev, stream, nullptr, 0};
        ++g_stream_scratch_count;
    }
    // grow: at least double, so a stream settles after a few calls
    int64_t bytes = slot->bytes * 2 > total ? slot->bytes * 2 : total;
    bytes = bytes < kStreamScratchMax ? bytes : kStreamScratchMax;
    uint8_t *p = nullptr;
    e = hipMallocAsync(reinterpret_cast<void **>(&p), static_cast<size_t>(bytes), stream);
    if (e != hipSuccess) return e;
    if (slot->ptr != nullptr) {
        e = hipFreeAsync(slot->ptr, stream);
        if (e != hipSuccess) {
            (void)hipFreeAsync(p, stream);
            return e;
        }
    }
    slot->ptr = p;
    slot->bytes = bytes;
    *out = p;
    return hipSuccess;
}

}  // namespace

hipError_t ws_acquire(Workspace &ws, int64_t total, hipStream_t stream, uint8_t **out, bool *owned) {
    *owned = false;
    *out = nullptr;
    if (ws.ptr != nullptr) {
        if (total > ws.bytes) return hipErrorInvalidValue;
        *out = ws.ptr;
        return hipSuccess;
    }
    hipError_t e = stream_scratch(total, stream, out);
    if (e != hipSuccess || *out != nullptr) return e;
    e = hipMallocAsync(reinterpret_cast<void **>(out), static_cast<size_t>(total), stream);
    *owned = e == hipSuccess;
    return e;
}

hipError_t ws_release(uint8_t *p, bool owned, hipStream_t stream) {
    return owned ? hipFreeAsync(p, stream) : hipSuccess;
}

hipError_t launch_copy(float *y, const float *src, int64_t count, hipStream_t stream) {
    if (count == 0 || y == src) return hipSuccess;
    const int64_t need = (count + 255) / 256;
    const int grid = static_cast<int>(need < 4096 ? need : 4096);
    hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, stream, y, src, count);
    return hipGetLastError();
}

}  // namespace q4k

// Scratch of q4k_gemv_batched_noalloc: one array per GPU, held from the
// library's load until the process ends.  Host code never uses this name as
// an address (on the host it is only a handle of the symbol): the device
// address comes from hipGetSymbolAddress, once per device.
static constexpr int64_t kStaticScratchBytes = int64_t{16} << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace q4k {
namespace {

std::mutex g_scratch_mutex;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device, looked up with that
// device current on its first use and kept.
hipError_t static_scratch(void **out) {
    *out = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace
}  // namespace q4k

using q4k::aligned;
using q4k::check_shape;
using q4k::from_hip;
using q4k::overlap;

extern "C" {

q4k_status q4k_gemv(const void *w, const float *x, float *y, int64_t n, int64_t k, void *stream) {
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (n == 0) return Q4K_OK;
    if (y == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(x, 4) || !aligned(y, 4)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(n) * 4, xb = static_cast<uint64_t>(k) * 4;
    if (overlap(y, yb, w, wb) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    return from_hip(q4k::launch_gemv(static_cast<const uint8_t *>(w), nullptr, x, nullptr, y, n, k,
                                     static_cast<hipStream_t>(stream)));
}

q4k_status q4k_gemv_dt(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype, int64_t n,
                       int64_t k, void *stream) {
    if ((x_dtype != Q4K_F32 && x_dtype != Q4K_F16) || (y_dtype != Q4K_F32 && y_dtype != Q4K_F16)) {
        return Q4K_ERR_INVALID_ARG;
    }
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (n == 0) return Q4K_OK;
    if (y == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    const uint64_t xe = x_dtype == Q4K_F16 ? 2 : 4, ye = y_dtype == Q4K_F16 ? 2 : 4;
    if (!aligned(w, 16) || !aligned(x, xe) || !aligned(y, ye)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(n) * ye, xb = static_cast<uint64_t>(k) * xe;
    if (overlap(y, yb, w, wb) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    return from_hip(q4k::launch_gemv_dt(static_cast<const uint8_t *>(w), x, x_dtype == Q4K_F16, y,
                                        y_dtype == Q4K_F16, n, k, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_gemv_residual(const void *w, const float *x, const float *r, float *y, int64_t n, int64_t k,
                             void *stream) {
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (n == 0) return Q4K_OK;
    if (y == nullptr || r == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(x, 4) || !aligned(y, 4) || !aligned(r, 4)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(n) * 4, xb = static_cast<uint64_t>(k) * 4;
    if (overlap(y, yb, w, wb) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    if (r != y && overlap(y, yb, r, yb)) return Q4K_ERR_INVALID_ARG;  // in place, or apart
    return from_hip(q4k::launch_gemv(static_cast<const uint8_t *>(w), nullptr, x, r, y, n, k,
                                     static_cast<hipStream_t>(stream)));
}

q4k_status q4k_gemv_multi(const q4k_gemv_item *items, int count, const float *x, int64_t k, void *stream) {
    if (count < 0 || count > Q4K_MAX_MULTI) return Q4K_ERR_INVALID_ARG;
    if (count == 0) return Q4K_OK;
    if (items == nullptr) return Q4K_ERR_INVALID_ARG;
    uint64_t wbytes[Q4K_MAX_MULTI];
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) {
        const q4k_status s = check_shape(items[i].n, k, &wbytes[i]);
        if (s != Q4K_OK) return s;
        const q4k_gemv_item &it = items[i];
        if (it.y_gate != nullptr && it.n != 0) {
            // per-head de-interleave: a power-of-two head size dividing n / 2
            const int64_t hd = it.head_dim;
            if (hd <= 0 || hd > (int64_t{1} << 30) || (hd & (hd - 1)) != 0) return Q4K_ERR_INVALID_ARG;
            if (it.n % (2 * hd) != 0) return Q4K_ERR_INVALID_ARG;
            if (k > 4096) return Q4K_ERR_UNSUPPORTED_SHAPE;  // one launch only up to k = 4096
        }
        rows += it.n;
    }
    if (rows == 0) return Q4K_OK;
    if (k > 0 && x == nullptr) return Q4K_ERR_INVALID_ARG;
    if (!aligned(x, 4)) return Q4K_ERR_MISALIGNED;
    const uint64_t xb = static_cast<uint64_t>(k) * 4;
    // every output range: y (all n rows, or the q half) and the gate half
    const void *out_p[2 * Q4K_MAX_MULTI];
    uint64_t out_b[2 * Q4K_MAX_MULTI];
    int nout = 0;
    q4k::GemvJob jobs[Q4K_MAX_MULTI];
    for (int i = 0; i < count; ++i) {
        const q4k_gemv_item &it = items[i];
        if (it.n == 0) {
            jobs[i] = q4k::GemvJob{nullptr, nullptr, nullptr, 0};
            continue;
        }
        const bool split = it.y_gate != nullptr;
        if (it.y == nullptr || (k > 0 && it.w == nullptr)) return Q4K_ERR_INVALID_ARG;
        if (!aligned(it.w, 16) || !aligned(it.y, 4) || !aligned(it.y_gate, 4)) return Q4K_ERR_MISALIGNED;
        const uint64_t yb = static_cast<uint64_t>(split ? it.n / 2 : it.n) * 4;
        out_p[nout] = it.y;
        out_b[nout++] = yb;
        if (split) {
            out_p[nout] = it.y_gate;
            out_b[nout++] = yb;
        }
        jobs[i] = q4k::GemvJob{static_cast<const uint8_t *>(it.w), it.y, nullptr, it.n};
        if (split) {
            jobs[i].y_gate = it.y_gate;
            int lg = 0;
            while ((int64_t{1} << lg) < it.head_dim) ++lg;
            jobs[i].head_log2 = lg;
        }
    }
    // no output may overlap x, any weight matrix or another output
    for (int a = 0; a < nout; ++a) {
        if (overlap(out_p[a], out_b[a], x, xb)) return Q4K_ERR_INVALID_ARG;
        for (int j = 0; j < count; ++j) {
            if (items[j].n != 0 && overlap(out_p[a], out_b[a], items[j].w, wbytes[j])) return Q4K_ERR_INVALID_ARG;
        }
        for (int b = a + 1; b < nout; ++b) {
            if (overlap(out_p[a], out_b[a], out_p[b], out_b[b])) return Q4K_ERR_INVALID_ARG;
        }
    }
    return from_hip(q4k::launch_gemv_multi(jobs, count, nullptr, x, k, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_q8_0_gemv(const void *w, const float *x, float *y, int64_t n, int64_t k, void *stream) {
    if (n < 0 || k < 0) return Q4K_ERR_INVALID_ARG;
    if (k % Q4K_Q8_0_BLOCK_WEIGHTS != 0) return Q4K_ERR_UNSUPPORTED_SHAPE;
    if (k > 0 && n > q4k::kMaxElems / k) return Q4K_ERR_INVALID_ARG;
    if (n == 0) return Q4K_OK;
    const uint64_t wb = static_cast<uint64_t>(n) * static_cast<uint64_t>(k / Q4K_Q8_0_BLOCK_WEIGHTS) *
                        Q4K_Q8_0_BLOCK_BYTES;
    if (y == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    if (!aligned(w, 2) || !aligned(x, 4) || !aligned(y, 4)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(n) * 4, xb = static_cast<uint64_t>(k) * 4;
    if (overlap(y, yb, w, wb) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    return from_hip(q4k::launch_q8_0_gemv(static_cast<const uint8_t *>(w), x, nullptr, y, n, k,
                                          static_cast<hipStream_t>(stream)));
}

q4k_status q4k_gemv_batched(const void *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                            void *stream) {
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (m < 0) return Q4K_ERR_INVALID_ARG;
    if (m > 0 && (n > q4k::kMaxElems / m || (k > 0 && m > q4k::kMaxElems / k))) return Q4K_ERR_INVALID_ARG;
    if (n == 0 || m == 0) return Q4K_OK;
    if (y == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(x, 4) || !aligned(y, 4)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(m) * n * 4, xb = static_cast<uint64_t>(m) * k * 4;
    if (overlap(y, yb, w, wb) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    return from_hip(q4k::launch_gemv_batched(static_cast<const uint8_t *>(w), x, y, m, n, k,
                                             static_cast<hipStream_t>(stream)));
}

namespace {

// Checks of q4k_gemv_batched_dt and its workspace form; on Q4K_OK with *run
// set the call has work to launch.
q4k_status check_batched(const void *w, const void *x, q4k_dtype x_dtype, const void *y, q4k_dtype y_dtype,
                         int64_t m, int64_t n, int64_t k, bool *run, uint64_t *w_bytes) {
    *run = false;
    if ((x_dtype != Q4K_F32 && x_dtype != Q4K_F16) || (y_dtype != Q4K_F32 && y_dtype != Q4K_F16)) {
        return Q4K_ERR_INVALID_ARG;
    }
    const q4k_status s = check_shape(n, k, w_bytes);
    if (s != Q4K_OK) return s;
    if (m < 0) return Q4K_ERR_INVALID_ARG;
    if (m > 0 && (n > q4k::kMaxElems / m || (k > 0 && m > q4k::kMaxElems / k))) return Q4K_ERR_INVALID_ARG;
    if (n == 0 || m == 0) return Q4K_OK;
    if (y == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    const uint64_t xe = x_dtype == Q4K_F16 ? 2 : 4, ye = y_dtype == Q4K_F16 ? 2 : 4;
    if (!aligned(w, 16) || !aligned(x, xe) || !aligned(y, ye)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(m) * n * ye, xb = static_cast<uint64_t>(m) * k * xe;
    if (overlap(y, yb, w, *w_bytes) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    *run = true;
    return Q4K_OK;
}

// Checks of q4k_prefill_gemm and its workspace form.
q4k_status check_prefill(const void *w, const void *x, const void *y, q4k_dtype y_dtype, int64_t m, int64_t n,
                         int64_t k, bool *run, uint64_t *w_bytes) {
    *run = false;
    if (y_dtype != Q4K_F32 && y_dtype != Q4K_F16) return Q4K_ERR_INVALID_ARG;
    const q4k_status s = check_shape(n, k, w_bytes);
    if (s != Q4K_OK) return s;
    // the kernel addresses one 128-row block of weights with 32-bit offsets
    if (k > (int64_t{1} << 24)) return Q4K_ERR_UNSUPPORTED_SHAPE;
    if (m < 0) return Q4K_ERR_INVALID_ARG;
    if (m > 0 && (n > q4k::kMaxElems / m || (k > 0 && m > q4k::kMaxElems / k))) return Q4K_ERR_INVALID_ARG;
    if (n == 0 || m == 0) return Q4K_OK;
    if (y == nullptr || (k > 0 && (w == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    const uint64_t ye = y_dtype == Q4K_F16 ? 2 : 4;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, ye)) return Q4K_ERR_MISALIGNED;
    const uint64_t yb = static_cast<uint64_t>(m) * n * ye, xb = static_cast<uint64_t>(m) * k * 2;
    if (overlap(y, yb, w, *w_bytes) || overlap(y, yb, x, xb)) return Q4K_ERR_INVALID_ARG;
    *run = true;
    return Q4K_OK;
}

// A caller's workspace, before its size is known: a non-negative size and,
// when given, 256-byte alignment.
q4k_status check_workspace_arg(const void *ws, int64_t ws_bytes) {
    if (ws_bytes < 0) return Q4K_ERR_INVALID_ARG;
    if (ws != nullptr && !aligned(ws, 256)) return Q4K_ERR_MISALIGNED;
    return Q4K_OK;
}

// ... and once the call's need is known: large enough, apart from w, x, y.
q4k_status check_workspace(const void *ws, int64_t ws_bytes, int64_t need, const void *w, uint64_t wb,
                           const void *x, uint64_t xb, const void *y, uint64_t yb) {
    if (need == 0) return Q4K_OK;
    if (ws == nullptr || ws_bytes < need) return Q4K_ERR_INVALID_ARG;
    const uint64_t b = static_cast<uint64_t>(need);
    if (overlap(ws, b, w, wb) || overlap(ws, b, x, xb) || overlap(ws, b, y, yb)) return Q4K_ERR_INVALID_ARG;
    return Q4K_OK;
}

}  // namespace

q4k_status q4k_gemv_batched_dt(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype,
                               int64_t m, int64_t n, int64_t k, void *stream) {
    bool run = false;
    uint64_t wb = 0;
    const q4k_status s = check_batched(w, x, x_dtype, y, y_dtype, m, n, k, &run, &wb);
    if (s != Q4K_OK || !run) return s;
    q4k::Workspace ws;
    return from_hip(q4k::launch_gemv_batched_dt(static_cast<const uint8_t *>(w), x, x_dtype == Q4K_F16, y,
                                                y_dtype == Q4K_F16, m, n, k, ws, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_gemv_batched_workspace_size(q4k_dtype x_dtype, q4k_dtype y_dtype, int64_t m, int64_t n, int64_t k,
                                           int64_t *bytes) {
    if (bytes == nullptr) return Q4K_ERR_INVALID_ARG;
    *bytes = 0;
    if ((x_dtype != Q4K_F32 && x_dtype != Q4K_F16) || (y_dtype != Q4K_F32 && y_dtype != Q4K_F16)) {
        return Q4K_ERR_INVALID_ARG;
    }
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (m < 0) return Q4K_ERR_INVALID_ARG;
    if (m > 0 && (n > q4k::kMaxElems / m || (k > 0 && m > q4k::kMaxElems / k))) return Q4K_ERR_INVALID_ARG;
    q4k::Workspace ws;
    ws.query = true;
    const hipError_t e = q4k::launch_gemv_batched_dt(nullptr, nullptr, x_dtype == Q4K_F16, nullptr,
                                                     y_dtype == Q4K_F16, m, n, k, ws, nullptr);
    if (e != hipSuccess) return Q4K_ERR_LAUNCH;
    *bytes = ws.need;
    return Q4K_OK;
}

q4k_status q4k_gemv_batched_ws(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype,
                               int64_t m, int64_t n, int64_t k, void *workspace, int64_t workspace_bytes,
                               void *stream) {
    bool run = false;
    uint64_t wb = 0;
    q4k_status s = check_batched(w, x, x_dtype, y, y_dtype, m, n, k, &run, &wb);
    if (s == Q4K_OK) s = check_workspace_arg(workspace, workspace_bytes);
    if (s != Q4K_OK || !run) return s;
    int64_t need = 0;
    s = q4k_gemv_batched_workspace_size(x_dtype, y_dtype, m, n, k, &need);
    if (s != Q4K_OK) return s;
    const uint64_t xe = x_dtype == Q4K_F16 ? 2 : 4, ye = y_dtype == Q4K_F16 ? 2 : 4;
    s = check_workspace(workspace, workspace_bytes, need, w, wb, x, static_cast<uint64_t>(m) * k * xe, y,
                        static_cast<uint64_t>(m) * n * ye);
    if (s != Q4K_OK) return s;
    q4k::Workspace ws;
    ws.ptr = static_cast<uint8_t *>(workspace);
    ws.bytes = workspace_bytes;
    return from_hip(q4k::launch_gemv_batched_dt(static_cast<const uint8_t *>(w), x, x_dtype == Q4K_F16, y,
                                                y_dtype == Q4K_F16, m, n, k, ws, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_gemv_batched_noalloc(const void *w, const void *x, q4k_dtype x_dtype, void *y, q4k_dtype y_dtype,
                                    int64_t m, int64_t n, int64_t k, void *stream) {
    bool run = false;
    uint64_t wb = 0;
    q4k_status s = check_batched(w, x, x_dtype, y, y_dtype, m, n, k, &run, &wb);
    if (s != Q4K_OK || !run) return s;
    int64_t need = 0;
    s = q4k_gemv_batched_workspace_size(x_dtype, y_dtype, m, n, k, &need);
    if (s != Q4K_OK) return s;
    if (need > kStaticScratchBytes) return Q4K_ERR_UNSUPPORTED_SHAPE;
    q4k::Workspace ws;
    if (need > 0) {
        void *p = nullptr;
        if (q4k::static_scratch(&p) != hipSuccess) return Q4K_ERR_LAUNCH;
        ws.ptr = static_cast<uint8_t *>(p);
        ws.bytes = kStaticScratchBytes;
    }
    return from_hip(q4k::launch_gemv_batched_dt(static_cast<const uint8_t *>(w), x, x_dtype == Q4K_F16, y,
                                                y_dtype == Q4K_F16, m, n, k, ws, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_prefill_gemm(const void *w, const void *x, void *y, q4k_dtype y_dtype, int64_t m, int64_t n,
                            int64_t k, void *stream) {
    bool run = false;
    uint64_t wb = 0;
    const q4k_status s = check_prefill(w, x, y, y_dtype, m, n, k, &run, &wb);
    if (s != Q4K_OK || !run) return s;
    q4k::Workspace ws;
    return from_hip(q4k::launch_prefill(static_cast<const uint8_t *>(w), static_cast<const _Float16 *>(x), y,
                                        y_dtype == Q4K_F16, m, n, k, ws, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_prefill_workspace_size(q4k_dtype y_dtype, int64_t m, int64_t n, int64_t k, int64_t *bytes) {
    if (bytes == nullptr) return Q4K_ERR_INVALID_ARG;
    *bytes = 0;
    if (y_dtype != Q4K_F32 && y_dtype != Q4K_F16) return Q4K_ERR_INVALID_ARG;
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (k > (int64_t{1} << 24)) return Q4K_ERR_UNSUPPORTED_SHAPE;
    if (m < 0) return Q4K_ERR_INVALID_ARG;
    if (m > 0 && (n > q4k::kMaxElems / m || (k > 0 && m > q4k::kMaxElems / k))) return Q4K_ERR_INVALID_ARG;
    q4k::Workspace ws;
    ws.query = true;
    const hipError_t e = q4k::launch_prefill(nullptr, nullptr, nullptr, y_dtype == Q4K_F16, m, n, k, ws, nullptr);
    if (e != hipSuccess) return Q4K_ERR_LAUNCH;
    *bytes = ws.need;
    return Q4K_OK;
}

q4k_status q4k_prefill_gemm_ws(const void *w, const void *x, void *y, q4k_dtype y_dtype, int64_t m, int64_t n,
                               int64_t k, void *workspace, int64_t workspace_bytes, void *stream) {
    bool run = false;
    uint64_t wb = 0;
    q4k_status s = check_prefill(w, x, y, y_dtype, m, n, k, &run, &wb);
    if (s == Q4K_OK) s = check_workspace_arg(workspace, workspace_bytes);
    if (s != Q4K_OK || !run) return s;
    int64_t need = 0;
    s = q4k_prefill_workspace_size(y_dtype, m, n, k, &need);
    if (s != Q4K_OK) return s;
    const uint64_t ye = y_dtype == Q4K_F16 ? 2 : 4;
    s = check_workspace(workspace, workspace_bytes, need, w, wb, x, static_cast<uint64_t>(m) * k * 2, y,
                        static_cast<uint64_t>(m) * n * ye);
    if (s != Q4K_OK) return s;
    q4k::Workspace ws;
    ws.ptr = static_cast<uint8_t *>(workspace);
    ws.bytes = workspace_bytes;
    return from_hip(q4k::launch_prefill(static_cast<const uint8_t *>(w), static_cast<const _Float16 *>(x), y,
                                        y_dtype == Q4K_F16, m, n, k, ws, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_fused_swiglu(const void *w_gate, const void *w_up, const float *x, float *h, int64_t n, int64_t k,
                            void *stream) {
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (n == 0) return Q4K_OK;
    if (h == nullptr || (k > 0 && (w_gate == nullptr || w_up == nullptr || x == nullptr))) return Q4K_ERR_INVALID_ARG;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(x, 4) || !aligned(h, 4)) return Q4K_ERR_MISALIGNED;
    const uint64_t hb = static_cast<uint64_t>(n) * 4, xb = static_cast<uint64_t>(k) * 4;
    if (overlap(h, hb, w_gate, wb) || overlap(h, hb, w_up, wb) || overlap(h, hb, x, xb)) return Q4K_ERR_INVALID_ARG;
    return from_hip(q4k::launch_gemv(static_cast<const uint8_t *>(w_gate), static_cast<const uint8_t *>(w_up), x,
                                     nullptr, h, n, k, static_cast<hipStream_t>(stream)));
}

q4k_status q4k_dequant(const void *w, float *out, int64_t n, int64_t k, void *stream) {
    uint64_t wb = 0;
    const q4k_status s = check_shape(n, k, &wb);
    if (s != Q4K_OK) return s;
    if (n == 0 || k == 0) return Q4K_OK;
    if (w == nullptr || out == nullptr) return Q4K_ERR_INVALID_ARG;
    if (!aligned(w, 16) || !aligned(out, 16)) return Q4K_ERR_MISALIGNED;
    const uint64_t ob = static_cast<uint64_t>(n) * k * 4;
    if (overlap(out, ob, w, wb)) return Q4K_ERR_INVALID_ARG;
    return from_hip(q4k::launch_dequant(static_cast<const uint8_t *>(w), out, n, k, static_cast<hipStream_t>(stream)));
}

const char *q4k_status_string(q4k_status s) {
    switch (s) {
        case Q4K_OK: return "ok";
        case Q4K_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, overlapping buffers or size overflow)";
        case Q4K_ERR_UNSUPPORTED_SHAPE:
            return "unsupported shape (k not a multiple of 256, or of 32 for Q8_0, or beyond a call's stated limits, "
                   "such as the 16 MiB of scratch of q4k_gemv_batched_noalloc)";
        case Q4K_ERR_MISALIGNED:
            return "misaligned pointer (w needs 16-byte alignment, activations/outputs their element size; dequant "
                   "output and workspaces as documented)";
        case Q4K_ERR_LAUNCH: return "kernel launch failed";
        default: break;  // any other int: the type spans the whole int range
    }
    return "unknown status";
}

int q4k_abi_version(void) { return Q4K_ABI_VERSION; }

}  // extern "C"
