"""Shared helpers of the GPU parity tests: device copies and the error bound.

The bound is the one the method states for every output:
    |y_gpu - y_ref| <= 2e-4 * sum_k |w_k x_k|
with y_ref and the magnitude sum from the f64 oracle.  Where the magnitude sum
is exactly zero the output must be exactly zero.
"""

from __future__ import annotations

import os

import numpy as np

REL = 2e-4
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def to_dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t):
    import torch

    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_bound(y_gpu, y_ref, a_ref, what: str, rel: float = REL) -> float:
    """Asserts the per-output bound; returns the worst error / magnitude-sum ratio."""
    y = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    a_ref = np.asarray(a_ref, dtype=np.float64)
    assert y.shape == y_ref.shape == a_ref.shape, (y.shape, y_ref.shape, a_ref.shape)
    err = np.abs(y - y_ref)
    zero = a_ref == 0
    ok = np.where(zero, y == 0, err <= rel * a_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(zero, np.where(y == 0, 0.0, np.inf), err / a_ref)
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {y.size} outputs outside {rel} * sum|w x|; "
                             f"worst ratio {worst:.3e}; first at {idx.tolist()}: gpu {y[tuple(idx[0])]!r} "
                             f"oracle {y_ref[tuple(idx[0])]!r} sum|wx| {a_ref[tuple(idx[0])]!r}")
    return worst


def check_swiglu_bound(h_gpu, ref: dict, what: str) -> float:
    """Bound on h = silu(g) u derived from the per-output GEMV bound on g and u:
    |dh| <= sup|silu'| eg (|u| + eu) + |silu(g)| eu + 8 ulp(h), sup|silu'| < 1.1."""
    h = np.asarray(h_gpu, dtype=np.float64)
    eg = REL * ref["ag"]
    eu = REL * ref["au"]
    g, u = ref["g"], ref["u"]
    silu_g = g / (1.0 + np.exp(-g))
    bound = 1.1 * eg * (np.abs(u) + eu) + np.abs(silu_g) * eu + 8 * 2.0 ** -24 * np.abs(ref["h"])
    err = np.abs(h - ref["h"])
    ok = err <= bound
    if not ok.all():
        i = int(np.argwhere(~ok)[0][0])
        raise AssertionError(f"{what}: {int((~ok).sum())} of {h.size} outputs outside the derived bound; first "
                             f"row {i}: gpu {h[i]!r} oracle {ref['h'][i]!r} bound {bound[i]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        return float(np.nanmax(np.where(bound > 0, err / bound, 0.0)))


def check_bound_f16(y16, y_ref, a_ref, what):
    """f16 output: the f32 bound widened by the output rounding.  An f32 result
    of magnitude >= 65520 rounds to +-inf: where the bound puts it surely
    there the output must be inf of the oracle's sign, where it may be on
    either side, inf of that sign is accepted too."""
    y = np.asarray(y16, dtype=np.float64)
    bound = REL * a_ref + 2.0 ** -11 * (np.abs(y_ref) + REL * a_ref) + 2.0 ** -25
    with np.errstate(invalid="ignore"):
        err = np.abs(y - y_ref)
    signed_inf = np.isinf(y) & (np.sign(y) == np.sign(y_ref))
    must_overflow = np.abs(y_ref) - REL * a_ref >= 65520.0
    may_overflow = np.abs(y_ref) + REL * a_ref >= 65520.0
    ok = np.where(must_overflow, signed_inf, (err <= bound) | (may_overflow & signed_inf))
    err = np.where(np.isinf(y), 0.0, err)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {y.size} f16 outputs outside the bound; first at "
                             f"{i.tolist()}: gpu {y[tuple(i)]!r} oracle {y_ref[tuple(i)]!r} bound {bound[tuple(i)]!r}")
    return float(np.max(err / bound)) if err.size else 0.0


def batched_on_gemv_kernels(m: int, n: int, k: int) -> bool:
    """Whether q4k_gemv_batched runs m tokens on the streaming GEMV kernels
    (token pairs, no scratch, each token bitwise equal to q4k_gemv) rather
    than on the matrix cores."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    few = (m <= 4 and k <= 4096) or (m == 2 and k <= 16384)
    many_rows = m > 2 and k <= 4096 and (n + 15) // 16 >= 4 * cus
    return m >= 2 and few and not many_rows
