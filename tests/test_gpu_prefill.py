"""GPU parity of the prefill GEMM (q4k_prefill_gemm: f16 activations, hundreds
of tokens, matrix cores) through the C ABI against the CPU oracle's batched
GEMM on the same activations (widened exactly to f32): every output within
2e-4 * sum|w x| (f32 output), plus the output rounding for f16 outputs.
Shapes cover ragged token and row tiles (m, n not multiples of 128), several
super-blocks, the 9B FFN shapes at prefill sizes (whole), special weight
values, and bitwise reruns.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import THREADS, check_bound, to_dev, to_host
from q4_dequant_gemv_amd import inputs
from test_gpu_dtypes import check_bound_f16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q4k():
    import torch

    from q4_dequant_gemv_amd import q4k as mod

    torch.cuda.init()
    mod.lib()
    oracle.build(force=False)
    return mod


def _report(name, worst):
    print(f"[parity] {name}: worst |err|/bound = {worst:.3e}", flush=True)


def _case(q4k, w, x16, label):
    import torch

    n = w.shape[0]
    m, k = x16.shape
    print(f"[case] prefill {label}: m={m} {n}x{k}", flush=True)
    wd, xd = to_dev(w.reshape(-1)), to_dev(x16)
    y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.prefill_gemm(wd, xd, y=y)
    y16 = q4k.prefill_gemm(wd, xd, out_dtype=torch.float16)
    again = q4k.prefill_gemm(wd, xd)
    torch.cuda.synchronize()
    assert torch.equal(y, again), f"{label}: two runs differ"
    assert torch.equal(y16, y.half()), f"{label}: f16 output is not the rounded f32 result"
    got = to_host(y)
    assert np.isfinite(got).all(), f"{label}: {int((~np.isfinite(got)).sum())} outputs not written"
    yr, ar = oracle.gemv_batched(w, x16.astype(np.float32), threads=THREADS)
    _report(label, check_bound(got, yr, ar, label))
    check_bound_f16(to_host(y16.float()), yr, ar, label + " f16")


@pytest.mark.parametrize("m,n,k", [(128, 128, 256), (130, 300, 512), (1, 64, 256), (127, 129, 1024), (256, 1024, 4096),
                                   (200, 257, 2304), (384, 640, 12288), (129, 131, 16384)])
def test_prefill_shapes(q4k, m, n, k):
    w = inputs.make_q4k(n, k, config_id=70, tensor_id=k)
    x16 = inputs.make_x(m, k, config_id=70, tensor_id=m).astype(np.float16)
    _case(q4k, w, x16, f"{m}x{n}x{k}")


@pytest.mark.parametrize("name,tid", [("gate_9b", 0), ("down_9b", 2)])
def test_prefill_9b_ffn_whole(q4k, name, tid):
    """512 tokens through the 9B gate and down projections, every output
    against the oracle."""
    n, k = inputs.SHAPES[name]
    m = 512
    w = inputs.make_q4k(n, k, config_id=71, tensor_id=tid)
    x16 = inputs.make_x(m, k, config_id=71, tensor_id=100 + tid).astype(np.float16)
    _case(q4k, w, x16, name)


def test_prefill_special_values(q4k):
    m, n, k = 160, 192, 1024
    x16 = inputs.make_x(m, k, config_id=72).astype(np.float16)
    # every weight exactly zero through cancellation (q = 1, sc = m, d = dmin)
    from independent_decoder import pack_scales

    blocks = inputs.make_q4k(n, k, config_id=72, tensor_id=1).reshape(-1, 144).copy()
    blocks[:, 16:] = 0x11
    blocks[:, 2:4] = blocks[:, 0:2]
    rng = np.random.default_rng(5)
    for b in blocks:
        v = list(rng.integers(1, 64, 8))
        b[4:16] = np.frombuffer(pack_scales(v, v), np.uint8)
    assert np.all(oracle.dequant(blocks.reshape(-1), k) == 0)
    y = to_host(q4k.prefill_gemm(to_dev(blocks.reshape(-1)), to_dev(x16), n=n))
    # the code and min terms cancel; what is left is rounding, bounded by the
    # size of the terms that cancel: sum |d sc q x| (the same blocks with dmin = 0)
    code_only = blocks.copy()
    code_only[:, 2:4] = 0
    _, a_code = oracle.gemv_batched(code_only.reshape(-1), x16.astype(np.float32), threads=THREADS)
    assert np.all(np.abs(y) <= 2e-4 * a_code)
    # zero codes: every weight is -dmin*m
    w = inputs.make_q4k(n, k, config_id=72, tensor_id=2).reshape(-1, 144).copy()
    w[:, 16:] = 0
    _case(q4k, w.reshape(n, -1), x16, "zero codes")
    # activations over the whole f16 range (large and subnormal values)
    xs = (x16.astype(np.float32) * np.exp2(rng.integers(-20, 12, (m, k)))).astype(np.float16)
    _case(q4k, inputs.make_q4k(n, k, config_id=72, tensor_id=3), xs, "wide x")
    # a NaN activation poisons its token's outputs only
    xn = x16.copy()
    xn[7, 100] = np.nan
    y = to_host(q4k.prefill_gemm(to_dev(inputs.make_q4k(n, k, config_id=72, tensor_id=3).reshape(-1)), to_dev(xn)))
    assert np.all(np.isnan(y[7])) and np.isfinite(np.delete(y, 7, axis=0)).all()


def test_prefill_k_zero(q4k):
    import torch

    y = torch.full((130, 10), 5.0, device="cuda")
    q4k.prefill_gemm(torch.empty(0, dtype=torch.uint8, device="cuda"),
                     torch.empty((130, 0), dtype=torch.float16, device="cuda"), y=y, n=10)
    assert np.all(to_host(y) == 0)
