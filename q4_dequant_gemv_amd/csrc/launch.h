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

// y[r] = sum_c W[r,c] x[c]; with w_up != nullptr computes
// h[r] = silu((W x)[r]) * (W_up x)[r] instead.
hipError_t launch_gemv(const uint8_t *w, const uint8_t *w_up, const float *x, float *y, int64_t n, int64_t k,
                       hipStream_t stream);

// y[t, r] = sum_c W[r,c] x[t,c] for t < m.
hipError_t launch_gemv_batched(const uint8_t *w, const float *x, float *y, int64_t m, int64_t n, int64_t k,
                               hipStream_t stream);

// Writes zeros to y[0..count) (the k == 0 empty sum).
hipError_t launch_fill_zero(float *y, int64_t count, hipStream_t stream);

}  // namespace q4k
