"""GPU parity of the Q8_0 GEMV (q4k_q8_0_gemv) through the C ABI against the
CPU oracle on the same seeded inputs: every output within
2e-4 * sum_k |w_k x_k|, every output, at small shapes and at the 9B shapes
(computed on the GPU in the configuration the benchmark times).  Shapes cover the streaming kernel (K % 64 == 0, K <= 4096), the
K-split kernel (K up to 16384), both with LDS-staged and register loads, and the one-wave-per-row kernel (an odd number
of blocks per row, a matrix that is only 2-byte aligned, K > 16384).
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import THREADS, check_bound, to_dev, to_host
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


def _report(name, worst):
    print(f"[parity] {name}: worst |err|/sum|wx| = {worst:.3e}", flush=True)


def _case(q4k, w, x, label):
    import torch

    n = w.shape[0]
    print(f"[case] q8_0 {label}: {n}x{x.size}", flush=True)
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    q4k.q8_0_gemv(to_dev(w.reshape(-1)), to_dev(x), y=y, n=n)
    got = to_host(y)
    assert np.isfinite(got).all() or not np.isfinite(x).all(), f"{label}: rows not written"
    yr, ar = oracle.q8_0_gemv(w, x, threads=THREADS)
    _report(f"q8_0 {label}", check_bound(got, yr, ar, label))
    return got


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (7, 64), (5, 320), (1024, 1024), (4097, 1024), (33, 2304),
                                 (300, 3072), (129, 4096), (65, 8192), (17, 12288), (8195, 12288), (9, 16384),
                                 (5, 20480), (3, 20512)])
def test_q8_0_shapes(q4k, n, k):
    w = inputs.make_q8_0(n, k, config_id=50, tensor_id=k)
    x = inputs.make_x(1, k, config_id=50, tensor_id=k)[0]
    _case(q4k, w, x, f"{n}x{k}")


@pytest.mark.parametrize("name,tid", [("q_proj_0p8b", 1), ("out_proj_0p8b", 2), ("gdn_qkv_0p8b", 3)])
def test_q8_0_0p8b_projections(q4k, name, tid):
    n, k = inputs.SHAPES[name]
    w = inputs.make_q8_0(n, k, config_id=51, tensor_id=tid)
    x = inputs.make_x(1, k, config_id=51, tensor_id=100 + tid)[0]
    _case(q4k, w, x, name)


@pytest.mark.parametrize("name,tid", [("lm_head_9b", 0), ("gate_9b", 1), ("down_9b", 2)])
def test_q8_0_9b_whole(q4k, name, tid):
    n, k = inputs.SHAPES[name]
    w = inputs.make_q8_0(n, k, config_id=52, tensor_id=tid)
    x = inputs.make_x(1, k, config_id=52, tensor_id=100 + tid)[0]
    _case(q4k, w, x, name)


def test_q8_0_two_byte_aligned_matrix(q4k):
    """A row range starting at an odd block (2-byte aligned pointer) takes the
    one-wave-per-row kernel and still matches the oracle."""
    import torch

    n, k = 64, 32 * 33  # 33 blocks per row: 1122-byte rows, every other row 2-byte aligned
    w = inputs.make_q8_0(n, k, config_id=53, tensor_id=0)
    x = inputs.make_x(1, k, config_id=53)[0]
    wd = to_dev(w.reshape(-1))
    rb = inputs.q8_0_row_bytes(k)
    y = torch.empty(n - 1, dtype=torch.float32, device="cuda")
    q4k.q8_0_gemv(wd[rb:], to_dev(x), y=y, n=n - 1)
    yr, ar = oracle.q8_0_gemv(w[1:], x, threads=THREADS)
    _report("q8_0 2-byte aligned", check_bound(to_host(y), yr, ar, "2-byte aligned"))


@pytest.mark.parametrize("n,k", [(300, 1024), (129, 4096), (17, 12288)])
def test_q8_0_staged_equals_register_path(q4k, n, k):
    """Rows of a multiple of 256 weights (K <= 4096, or 8192 < K <= 12288) in a
    16-byte aligned matrix stream through LDS; the same bytes at an address
    that is 4-byte but not 16-byte aligned stream through registers.  Both give
    bitwise the same outputs, inside the oracle's bound."""
    import torch

    print(f"[case] q8_0 staged vs register loads {n}x{k}", flush=True)
    w = inputs.make_q8_0(n, k, config_id=56, tensor_id=k)
    x = inputs.make_x(1, k, config_id=56, tensor_id=k)[0]
    flat = w.reshape(-1)
    wa = to_dev(flat)
    assert wa.data_ptr() % 16 == 0
    buf = torch.zeros(flat.size + 16, dtype=torch.uint8, device="cuda")
    buf[4:4 + flat.size].copy_(wa)
    w4 = buf[4:4 + flat.size]
    assert w4.data_ptr() % 16 == 4
    xd = to_dev(x)
    ya = q4k.q8_0_gemv(wa, xd, n=n)
    y4 = q4k.q8_0_gemv(w4, xd, n=n)
    assert torch.equal(ya, y4)
    yr, ar = oracle.q8_0_gemv(w, x, threads=THREADS)
    _report(f"q8_0 staged {n}x{k}", check_bound(to_host(ya), yr, ar, "staged"))


def test_q8_0_special_values(q4k):
    n, k = 64, 1024
    x = inputs.make_x(1, k, config_id=54)[0]
    g = np.random.default_rng(55)
    # every code -128 (the one value without a positive counterpart)
    q = np.full((n * k // 32, 32), -128, np.int8)
    d = g.uniform(1e-4, 1e-3, n * k // 32).astype(np.float16)
    _case(q4k, inputs.assemble_q8_0(q, d).reshape(n, -1), x, "all -128")
    # d = 0 everywhere gives exactly 0; x = 0 gives exactly 0
    w = inputs.assemble_q8_0(g.integers(-127, 128, (n * k // 32, 32), dtype=np.int8),
                             np.zeros(n * k // 32, np.float16)).reshape(n, -1)
    assert np.all(to_host(q4k.q8_0_gemv(to_dev(w.reshape(-1)), to_dev(x), n=n)) == 0)
    w = inputs.make_q8_0(n, k, config_id=54, tensor_id=1)
    assert np.all(to_host(q4k.q8_0_gemv(to_dev(w.reshape(-1)), to_dev(np.zeros(k, np.float32)), n=n)) == 0)
    # arbitrary finite f16 d of both signs (subnormals included)
    bits = g.integers(0, 0x7800, size=n * k // 32, dtype=np.uint16) | (
        g.integers(0, 2, size=n * k // 32, dtype=np.uint16) << 15)
    wb = inputs.assemble_q8_0(g.integers(-128, 128, (n * k // 32, 32), dtype=np.int8),
                              bits.view(np.float16)).reshape(n, -1)
    _case(q4k, wb, x, "f16 range")
    # activations spanning 16 binades, and tiny / huge scales
    xs = (x * np.exp2(g.integers(-8, 9, k))).astype(np.float32)
    _case(q4k, w, xs, "wide x")
    for s in (1e-30, 1e25):
        _case(q4k, w, (x * np.float32(s)).astype(np.float32), f"x*{s}")
    # a non-finite activation poisons every output
    xn = x.copy()
    xn[5] = np.nan
    y = to_host(q4k.q8_0_gemv(to_dev(w.reshape(-1)), to_dev(xn), n=n))
    assert np.all(np.isnan(y))


def test_q8_0_deterministic_and_k_zero(q4k):
    import torch

    n, k = 2048, 4096
    wd = to_dev(inputs.make_q8_0(n, k, config_id=56, tensor_id=0).reshape(-1))
    xd = to_dev(inputs.make_x(1, k, config_id=56)[0])
    base = to_host(q4k.q8_0_gemv(wd, xd))
    for _ in range(3):
        np.testing.assert_array_equal(to_host(q4k.q8_0_gemv(wd, xd)), base)
    y = torch.full((10,), 5.0, device="cuda")
    q4k.q8_0_gemv(torch.empty(0, dtype=torch.uint8, device="cuda"), torch.empty(0, device="cuda"), y=y, n=10)
    assert np.all(to_host(y) == 0)
