"""GPU parity of the f16 activation / f16 output variants (q4k_gemv_dt,
q4k_gemv_batched_dt) through the C ABI.

Checks, on the same seeded inputs:
  * f16 activations are widened exactly, so every result equals, bit for bit,
    the f32 call on those widened values;
  * an f16 output is the f32 result rounded to nearest even, so it equals,
    bit for bit, the f32 call's output rounded by torch (where K is not split
    across workgroups; with the split, whose f32 atomics may add in any order,
    the f16 output is checked against the bound below instead);
  * against the oracle (on the widened activations): within
    2e-4 * sum|w x| for f32 outputs, plus the f16 rounding of the output
    (2^-11 of |y|, 2^-25 in the subnormal range) for f16 outputs.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import REL, THREADS, batched_on_gemv_kernels, check_bound, check_bound_f16, to_dev, to_host
from q4_dequant_gemv_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    import torch

    from q4_dequant_gemv_amd import q4k as mod

    torch.cuda.init()
    mod.lib()
    oracle.build(force=False)
    return mod


def _f16_x(m, k, cfg, tid):
    # activations rounded to f16 once; the oracle sees exactly these values
    return inputs.make_x(m, k, config_id=cfg, tensor_id=tid).astype(np.float16)


@pytest.mark.parametrize("n,k", [(1024, 1024), (4097, 1024), (33, 2304), (129, 4096), (65, 12288), (9, 16384),
                                 (5, 20480)])
def test_gemv_dt_all_combinations(q4k, n, k):
    import torch

    w = inputs.make_q4k(n, k, config_id=60, tensor_id=k)
    x16 = _f16_x(1, k, 60, k)[0]
    wd = to_dev(w.reshape(-1))
    xh = to_dev(x16)
    xf = xh.float()
    print(f"[case] gemv_dt {n}x{k}", flush=True)
    ref32 = q4k.gemv(wd, xf)                       # the f32 path on the widened activations
    out = {}
    for xd in ("f16", "f32"):
        for yd in ("f16", "f32"):
            y = torch.full((n,), float("nan"), dtype=torch.float16 if yd == "f16" else torch.float32, device="cuda")
            q4k.gemv_dt(wd, xh if xd == "f16" else xf, y=y)
            out[(xd, yd)] = y
    torch.cuda.synchronize()
    for xd in ("f16", "f32"):
        assert torch.equal(out[(xd, "f32")], ref32), f"x {xd}: f32 output differs from the f32 path"
        assert torch.equal(out[(xd, "f16")], ref32.half()), f"x {xd}: f16 output is not the rounded f32 result"
    yr, ar = oracle.gemv(w, x16.astype(np.float32), threads=THREADS)
    check_bound(to_host(out[("f16", "f32")]), yr, ar, f"gemv_dt {n}x{k} f16->f32")
    check_bound_f16(to_host(out[("f16", "f16")].float()), yr, ar, f"gemv_dt {n}x{k} f16->f16")


def test_gemv_dt_full_size_lm_head_9b(q4k):
    """The 9B lm_head with f16 activations and f16 logits, every row against
    the oracle."""
    import torch

    n, k = inputs.SHAPES["lm_head_9b"]
    w = inputs.make_q4k(n, k, config_id=61, tensor_id=0)
    x16 = _f16_x(1, k, 61, 100)[0]
    y = torch.full((n,), float("nan"), dtype=torch.float16, device="cuda")
    q4k.gemv_dt(to_dev(w.reshape(-1)), to_dev(x16), y=y)
    got = to_host(y.float())
    assert np.isfinite(got).all()
    yr, ar = oracle.gemv(w, x16.astype(np.float32), threads=THREADS)
    check_bound_f16(got, yr, ar, "lm_head 9b f16->f16")


def test_gemv_dt_two_byte_aligned_f16_and_overflow(q4k):
    import torch

    n, k = 256, 4096
    w = inputs.make_q4k(n, k, config_id=62, tensor_id=0)
    wd = to_dev(w.reshape(-1))
    x16 = _f16_x(1, k + 1, 62, 0)[0]
    big = to_dev(x16)
    xv = big[1:]                      # an f16 vector that starts 2 bytes into an allocation
    assert xv.data_ptr() % 4 == 2
    y = q4k.gemv_dt(wd, xv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, q4k.gemv(wd, xv.float().contiguous()))
    # outputs beyond the f16 range become +-inf, the rest stay finite
    xs = to_dev((x16[1:].astype(np.float32) * 3000.0).astype(np.float16))
    y16 = to_host(q4k.gemv_dt(wd, xs).float())
    yr, ar = oracle.gemv(w, (x16[1:].astype(np.float32) * 3000.0).astype(np.float16).astype(np.float32),
                         threads=THREADS)
    over = np.abs(yr) - REL * ar > 65520.0
    under = np.abs(yr) + REL * ar < 65504.0
    assert over.any() and under.any()
    assert np.all(np.isinf(y16[over]) & (np.sign(y16[over]) == np.sign(yr[over])))
    assert np.all(np.isfinite(y16[under]))


@pytest.mark.parametrize("m,n,k", [(2, 300, 2048), (16, 4096, 1024), (33, 513, 1024), (64, 4100, 2048),
                                   (100, 700, 2304), (4, 70, 12288), (40, 70, 4096), (17, 4096, 4096),
                                   (2, 70, 12288), (3, 513, 1024), (4, 1000, 4096), (16, 4100, 2304),
                                   (6, 4096, 1024)])
def test_batched_dt_all_combinations(q4k, m, n, k):
    import torch

    w = inputs.make_q4k(n, k, config_id=63, tensor_id=k)
    x16 = _f16_x(m, k, 63, m)
    wd = to_dev(w.reshape(-1))
    xh = to_dev(x16)
    xf = xh.float()
    print(f"[case] batched_dt m={m} {n}x{k}", flush=True)
    yr, ar = oracle.gemv_batched(w, x16.astype(np.float32), threads=THREADS)
    # few rows per CU on the matrix-core kernel: K is split across workgroups
    # and added with atomics (a few tokens run on the streaming kernels instead)
    streaming = batched_on_gemv_kernels(m, n, k)
    split = not streaming and n < 16 * torch.cuda.get_device_properties(0).multi_processor_count and k >= 512
    for xd in ("f16", "f32"):
        xin = xh if xd == "f16" else xf
        y32 = q4k.gemv_batched_dt(wd, xin, out_dtype=torch.float32)
        y16 = q4k.gemv_batched_dt(wd, xin, out_dtype=torch.float16)
        torch.cuda.synchronize()
        check_bound(to_host(y32), yr, ar, f"batched_dt m={m} {n}x{k} {xd}->f32")
        check_bound_f16(to_host(y16.float()), yr, ar, f"batched_dt m={m} {n}x{k} {xd}->f16")
        if not split:
            assert torch.equal(y32, q4k.gemv_batched(wd, xf)), f"{xd}: f32 output differs from the f32 path"
            assert torch.equal(y16, y32.half()), f"{xd}: f16 output is not the rounded f32 result"


@pytest.mark.parametrize("m,n,k", [(128, 1024, 2048), (300, 700, 4096), (129, 96, 12288)])
def test_batched_dt_f16_prefill_sizes_route_to_prefill(q4k, m, n, k):
    """f16 activations at m >= 128 (16-byte aligned): the batched call runs the
    prefill GEMM, so it equals q4k_prefill_gemm bit for bit (also through a
    workspace of the queried size), and stays inside the oracle's bound.  An
    x that is only 2-byte aligned takes the skinny-GEMM path, also inside the
    bound, with the same workspace size."""
    import torch

    w = inputs.make_q4k(n, k, config_id=64, tensor_id=k)
    x16 = _f16_x(m, k, 64, m)
    wd, xh = to_dev(w.reshape(-1)), to_dev(x16)
    assert xh.data_ptr() % 16 == 0
    print(f"[case] batched_dt f16 m={m} {n}x{k}", flush=True)
    for yd in (torch.float32, torch.float16):
        yb = q4k.gemv_batched_dt(wd, xh, out_dtype=yd)
        yp = q4k.prefill_gemm(wd, xh, out_dtype=yd)
        torch.cuda.synchronize()
        assert torch.equal(yb, yp), "f16 batched call at prefill sizes differs from the prefill GEMM"
    need = q4k.gemv_batched_workspace_size(m, n, k, x_dtype=torch.float16, out_dtype=torch.float32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    yw = q4k.gemv_batched_ws(wd, xh, ws, out_dtype=torch.float32)
    assert torch.equal(yw, q4k.prefill_gemm(wd, xh, out_dtype=torch.float32))
    yr, ar = oracle.gemv_batched(w, x16.astype(np.float32), threads=THREADS)
    check_bound(to_host(yw), yr, ar, f"batched_dt f16 m={m} {n}x{k} (prefill)")
    # the same activations 2 bytes into an allocation: the skinny-GEMM path
    big = torch.empty(m * k + 1, dtype=torch.float16, device="cuda")
    xv = big[1:].view(m, k)
    xv.copy_(xh)
    assert xv.data_ptr() % 16 == 2
    y2 = q4k.gemv_batched_ws(wd, xv, ws, out_dtype=torch.float32)
    check_bound(to_host(y2), yr, ar, f"batched_dt f16 m={m} {n}x{k} (2-byte aligned x)")


def test_batched_dt_k_zero(q4k):
    import torch

    y = torch.full((3, 10), 5.0, dtype=torch.float16, device="cuda")
    q4k.gemv_batched_dt(torch.empty(0, dtype=torch.uint8, device="cuda"),
                        torch.empty((3, 0), dtype=torch.float16, device="cuda"), y=y, n=10)
    assert np.all(to_host(y.float()) == 0)
    y1 = torch.full((10,), 5.0, dtype=torch.float16, device="cuda")
    q4k.gemv_dt(torch.empty(0, dtype=torch.uint8, device="cuda"), torch.empty(0, dtype=torch.float16, device="cuda"),
                y=y1, n=10)
    assert np.all(to_host(y1.float()) == 0)
