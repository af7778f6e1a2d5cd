// Host-side launchers of the Q4_K kernels (internal to libq4k.so).  Each
// launcher assumes its arguments were validated by the C ABI layer (api.hip)
// and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

// Compute units of the current device, cached per device.
int device_cu_count();

hipError_t launch_dequant(const uint8_t *w, float *out, int64_t n, int64_t k, hipStream_t stream);

// Device scratch of one call.  ptr != nullptr: the caller's buffer of `bytes`
// (hipErrorInvalidValue if the call needs more); ptr == nullptr: taken
// stream-ordered for the call (hipMallocAsync / hipFreeAsync).  query: nothing
// is launched and `need` receives the largest block the call would use (the
// launches of one call run in order on one stream, so they share it).
struct Workspace {
    uint8_t *ptr = nullptr;
    int64_t bytes = 0;
    bool query = false;
    int64_t need = 0;
};

// Takes `total` bytes of ws for a launch sequence (not in query mode): *out,
// and *owned if they were allocated here (give them back with ws_release).
hipError_t ws_acquire(Workspace &ws, int64_t total, hipStream_t stream, uint8_t **out, bool *owned);
hipError_t ws_release(uint8_t *p, bool owned, hipStream_t stream);

// One matrix of a batch-1 GEMV launch: y[i] = sum_c W[i,c] x[c] (+ r[i] if
// r != nullptr; r may equal y).
struct GemvJob {
    const uint8_t *w;
    void *y;  // f32 [n] (f16 for launch_gemv_dt with y_f16)
    const float *r;
    int64_t n;
    // Per-head de-interleave of the output (q and gate halves of each head):
    // with y_gate set, row r = h*2D + j (D = 2^head_log2) goes to y[h*D + j]
    // if j < D, else to y_gate[h*D + j - D].  kPlainHead: every row r to y[r].
    void *y_gate = nullptr;
    int head_log2 = kPlainHead;
    static constexpr int kPlainHead = 61;
};

// y[i] = sum_c W[i,c] x[c] (+ r[i]); with w_up != nullptr computes
// h[i] = silu((W x)[i]) * (W_up x)[i] instead (r must be null then).
hipError_t launch_gemv(const uint8_t *w, const uint8_t *w_up, const float *x, const float *r, float *y, int64_t n,
                       int64_t k, hipStream_t stream);

// Up to 8 matrices with the same k against one x; those with k/64 <= 64
// groups share one launch.
hipError_t launch_gemv_multi(const GemvJob *jobs, int count, const uint8_t *w_up, const float *x, int64_t k,
                             hipStream_t stream);

// Batch-1 GEMV with f16 or f32 activations (x_f16) and outputs (y_f16); f16
// activations are widened exactly, outputs rounded to nearest even.
hipError_t launch_gemv_dt(const uint8_t *w, const void *x, bool x_f16, void *y, bool y_f16, int64_t n, int64_t k,
                          hipStream_t stream);

// Q8_0 weights (34-byte blocks of 32): y[i] = sum_c W[i,c] x[c] (+ r[i]).
hipError_t launch_q8_0_gemv(const uint8_t *w, const float *x, const float *r, float *y, int64_t n, int64_t k,
                            hipStream_t stream);

// Small batches on the streaming GEMV kernels: y[t, r] = sum_c W[r,c] x[t,c]
// for 2 <= m <= kTokensMax tokens with k <= kTokensMaxK, or m == 2 with
// k <= kTokensSplitMaxK (the K-split kernel); f16 or f32 x and y.
constexpr int64_t kTokensMax = 4;
constexpr int64_t kTokensMaxK = 4096;
constexpr int64_t kTokensSplitMaxK = 16384;
hipError_t launch_gemv_tokens(const uint8_t *w, const void *x, bool x_f16, void *y, bool y_f16, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream);

// y[t, r] = sum_c W[r,c] x[t,c] for t < m.
hipError_t launch_gemv_batched(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                               hipStream_t stream);

// The same with f16 or f32 activations and outputs.
hipError_t launch_gemv_batched_dt(const uint8_t *w, const void *x, bool x_f16, void *y, bool y_f16, int64_t m,
                                  int64_t n, int64_t k, Workspace &ws, hipStream_t stream);

// Prefill-size GEMM with f16 activations: y[t, r] = sum_c W[r,c] x[t,c],
// x f16 [m, k] (16-byte aligned), y f32 or f16 [m, n].
hipError_t launch_prefill(const uint8_t *w, const _Float16 *x, void *y, bool y_f16, int64_t m, int64_t n, int64_t k,
                          Workspace &ws, hipStream_t stream);
// The batched call with f16 activations hands m >= kPrefillMinTokens tokens
// (16-byte aligned x, k <= kPrefillMaxK) to the prefill GEMM.
constexpr int64_t kPrefillMinTokens = 128;
constexpr int64_t kPrefillMaxK = int64_t{1} << 24;

// Writes zeros to y[0..count) (the k == 0 empty sum).
hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream);
hipError_t launch_fill_zero_f16(_Float16 *y, int64_t count, hipStream_t stream);

// y[0..count) = src[0..count) (the k == 0 sum plus a residual; src may equal y).
hipError_t launch_copy(float *y, const float *src, int64_t count, hipStream_t stream);

}  // namespace q4k
