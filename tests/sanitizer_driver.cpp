// Host-side checks of the C ABI's argument validation, built together with
// libq4k's sources under AddressSanitizer and UndefinedBehaviorSanitizer
// (host code only) by tests/test_sanitizers_cpu.py.  Every call here must be
// refused, or be an empty call, before anything reaches the GPU: the device
// addresses are fake and never dereferenced, and no GPU is needed.  Sizes at
// the edges of int64 exercise the overflow checks, where a wrapped product
// would be undefined behaviour.  Exit status 0: every status as expected.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "q4k.h"

namespace {

int failures = 0;

void expect(const char *what, q4k_status got, q4k_status want) {
    if (got != want) {
        ++failures;
        fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, static_cast<int>(got), static_cast<int>(want));
    }
}

void *at(uintptr_t a) { return reinterpret_cast<void *>(a); }

const uintptr_t A = 0x7F0000000000ull;
const uintptr_t W = A, X = A + 0x10000000, Y = A + 0x20000000, R = A + 0x30000000, WS = A + 0x40000000;
const int64_t kBig = INT64_MAX;

}  // namespace

int main() {
    const q4k_status OK = Q4K_OK, INV = Q4K_ERR_INVALID_ARG, SHAPE = Q4K_ERR_UNSUPPORTED_SHAPE,
                     MIS = Q4K_ERR_MISALIGNED;
    float *x = static_cast<float *>(at(X));
    float *y = static_cast<float *>(at(Y));

    // q4k_gemv
    expect("gemv k%256", q4k_gemv(at(W), x, y, 16, 300, nullptr), SHAPE);
    expect("gemv n<0", q4k_gemv(at(W), x, y, -1, 256, nullptr), INV);
    expect("gemv null w", q4k_gemv(nullptr, x, y, 16, 256, nullptr), INV);
    expect("gemv w align", q4k_gemv(at(W + 8), x, y, 16, 256, nullptr), MIS);
    expect("gemv y overlaps w", q4k_gemv(at(W), x, static_cast<float *>(at(W + 64)), 16, 256, nullptr), INV);
    expect("gemv n*k overflow", q4k_gemv(at(W), x, y, int64_t{1} << 50, int64_t{1} << 20, nullptr), INV);
    expect("gemv n max", q4k_gemv(at(W), x, y, kBig, 256, nullptr), INV);
    expect("gemv k max", q4k_gemv(at(W), x, y, 16, kBig - kBig % 256, nullptr), INV);
    expect("gemv empty", q4k_gemv(at(W), x, y, 0, 256, nullptr), OK);

    // q4k_gemv_dt
    expect("gemv_dt dtype", q4k_gemv_dt(at(W), x, static_cast<q4k_dtype>(2), y, Q4K_F32, 16, 256, nullptr), INV);
    expect("gemv_dt f16 x align", q4k_gemv_dt(at(W), at(X + 1), Q4K_F16, y, Q4K_F16, 16, 256, nullptr), MIS);
    expect("gemv_dt overflow", q4k_gemv_dt(at(W), x, Q4K_F16, y, Q4K_F16, kBig, kBig - kBig % 256, nullptr), INV);

    // q4k_gemv_residual
    expect("residual null r", q4k_gemv_residual(at(W), x, nullptr, y, 16, 256, nullptr), INV);
    expect("residual r overlaps y", q4k_gemv_residual(at(W), x, static_cast<float *>(at(Y + 4)), y, 16, 256, nullptr),
           INV);
    expect("residual overflow", q4k_gemv_residual(at(W), x, static_cast<float *>(at(R)), y, kBig, 256, nullptr), INV);

    // q4k_gemv_multi
    q4k_gemv_item items[Q4K_MAX_MULTI + 1];
    memset(items, 0, sizeof(items));
    for (int i = 0; i <= Q4K_MAX_MULTI; ++i) {
        items[i].w = at(W + static_cast<uintptr_t>(i) * 0x1000000);
        items[i].y = static_cast<float *>(at(Y + static_cast<uintptr_t>(i) * 0x100000));
        items[i].n = 16;
    }
    expect("multi count", q4k_gemv_multi(items, Q4K_MAX_MULTI + 1, x, 256, nullptr), INV);
    expect("multi count<0", q4k_gemv_multi(items, -1, x, 256, nullptr), INV);
    expect("multi null items", q4k_gemv_multi(nullptr, 2, x, 256, nullptr), INV);
    items[1].y = items[0].y + 8;  // two outputs overlap
    expect("multi outputs overlap", q4k_gemv_multi(items, 2, x, 256, nullptr), INV);
    items[1].y = static_cast<float *>(at(Y + 0x100000));
    items[1].n = kBig;
    expect("multi overflow", q4k_gemv_multi(items, 2, x, 256, nullptr), INV);
    items[1].n = 16;
    items[0].y_gate = static_cast<float *>(at(Y + 0x800000));
    items[0].head_dim = 3;  // not a power of two
    expect("multi head_dim", q4k_gemv_multi(items, 1, x, 256, nullptr), INV);
    items[0].head_dim = int64_t{1} << 62;
    expect("multi head_dim huge", q4k_gemv_multi(items, 1, x, 256, nullptr), INV);
    items[0].y_gate = nullptr;
    expect("multi empty", q4k_gemv_multi(items, 0, x, 256, nullptr), OK);

    // q4k_q8_0_gemv
    expect("q8_0 k%32", q4k_q8_0_gemv(at(W), x, y, 16, 48, nullptr), SHAPE);
    expect("q8_0 overflow", q4k_q8_0_gemv(at(W), x, y, kBig, 64, nullptr), INV);

    // batched, batched_dt, prefill
    expect("batched m<0", q4k_gemv_batched(at(W), x, y, -1, 16, 256, nullptr), INV);
    expect("batched overflow m*n", q4k_gemv_batched(at(W), x, y, kBig, kBig, 256, nullptr), INV);
    expect("batched overflow m*k", q4k_gemv_batched(at(W), x, y, int64_t{1} << 40, 16, int64_t{1} << 40, nullptr),
           INV);
    expect("batched empty", q4k_gemv_batched(at(W), x, y, 0, 16, 256, nullptr), OK);
    expect("batched_dt dtype",
           q4k_gemv_batched_dt(at(W), x, Q4K_F32, y, static_cast<q4k_dtype>(-1), 4, 16, 256, nullptr), INV);
    expect("prefill k max", q4k_prefill_gemm(at(W), x, y, Q4K_F32, 128, 16, (int64_t{1} << 24) + 256, nullptr),
           SHAPE);
    expect("prefill overflow", q4k_prefill_gemm(at(W), x, y, Q4K_F32, kBig, 16, 256, nullptr), INV);

    // workspace queries and the _ws forms
    int64_t bytes = -1;
    expect("ws size null out", q4k_gemv_batched_workspace_size(Q4K_F32, Q4K_F32, 4, 16, 256, nullptr), INV);
    expect("ws size one token", q4k_gemv_batched_workspace_size(Q4K_F32, Q4K_F32, 1, 4096, 4096, &bytes), OK);
    if (bytes != 0) {
        ++failures;
        fprintf(stderr, "FAIL ws size one token: %lld bytes\n", static_cast<long long>(bytes));
    }
    expect("ws size overflow", q4k_gemv_batched_workspace_size(Q4K_F32, Q4K_F32, kBig, kBig, 256, &bytes), INV);
    expect("prefill ws size overflow", q4k_prefill_workspace_size(Q4K_F32, kBig, 16, 256, &bytes), INV);
    expect("batched_ws misaligned workspace",
           q4k_gemv_batched_ws(at(W), x, Q4K_F32, y, Q4K_F32, 64, 4096, 1024, at(WS + 16), int64_t{1} << 30, nullptr),
           MIS);
    expect("batched_ws negative bytes",
           q4k_gemv_batched_ws(at(W), x, Q4K_F32, y, Q4K_F32, 64, 4096, 1024, at(WS), -1, nullptr), INV);

    // swiglu and dequant
    expect("swiglu null up", q4k_fused_swiglu(at(W), nullptr, x, y, 16, 256, nullptr), INV);
    expect("swiglu overflow", q4k_fused_swiglu(at(W), at(R), x, y, kBig, 256, nullptr), INV);
    expect("dequant k%256", q4k_dequant(at(W), y, 16, 300, nullptr), SHAPE);
    expect("dequant overflow", q4k_dequant(at(W), y, kBig, 256, nullptr), INV);
    expect("dequant out align", q4k_dequant(at(W), static_cast<float *>(at(Y + 4)), 16, 256, nullptr), MIS);

    // strings and version
    for (int s = 0; s <= 4; ++s) {
        if (q4k_status_string(static_cast<q4k_status>(s)) == nullptr) ++failures;
    }
    if (strcmp(q4k_status_string(static_cast<q4k_status>(99)), "unknown status") != 0) ++failures;
    if (q4k_abi_version() != Q4K_ABI_VERSION) ++failures;

    if (failures != 0) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitizer driver: all checks passed\n");
    return 0;
}
