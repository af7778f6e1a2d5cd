"""q4k_gemv_batched_noalloc (the batched call with its scratch in the
library's per-GPU array, for callers that cannot allocate) against
q4k_gemv_batched_ws (the same call with a caller workspace), through the C
ABI, on two calls in a row, the second with a smaller input: bitwise equal
where the call is reproducible (at least 16 rows per compute unit), and both
inside the oracle's bound."""

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


def _cus():
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


def _case(q4k, m, n, k, seed, x_dtype, reproducible):
    import torch

    print(f"[case] noalloc m={m} {n}x{k} x={x_dtype}", flush=True)
    wh = inputs.make_q4k(n, k, config_id=80, tensor_id=seed)
    xh = inputs.make_x(m, k, config_id=80, tensor_id=seed)
    w = to_dev(wh.reshape(-1))
    x = to_dev(xh).to(x_dtype)
    need = q4k.gemv_batched_workspace_size(m, n, k, x_dtype=x_dtype, out_dtype=torch.float32)
    assert 0 < need <= q4k.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y_ws = torch.empty((m, n), dtype=torch.float32, device="cuda")
    y_na = torch.full((m, n), np.nan, dtype=torch.float32, device="cuda")
    q4k.gemv_batched_ws(w, x, ws, y=y_ws)
    q4k.gemv_batched_noalloc(w, x, y=y_na)
    a, b = to_host(y_ws), to_host(y_na)
    if reproducible:
        np.testing.assert_array_equal(a, b)
    yr, ar = oracle.gemv_batched(wh, x.float().cpu().numpy(), threads=THREADS)
    check_bound(a, yr, ar, f"workspace form m={m}")
    check_bound(b, yr, ar, f"no-allocation form m={m}")


def test_noalloc_equals_workspace_form_two_calls(q4k):
    import torch

    n_big = 16 * _cus()
    # first call: 64 tokens over a row tile per CU (staged matrix-core kernel,
    # bitwise reproducible); second, smaller: 16 tokens over 512 rows at
    # k = 1024 (K split across workgroups: inside the bound)
    _case(q4k, 64, n_big, 4096, seed=1, x_dtype=torch.float32, reproducible=True)
    _case(q4k, 16, 512, 1024, seed=2, x_dtype=torch.float32, reproducible=False)


def test_noalloc_again_after_other_calls(q4k):
    """The array keeps the previous call's contents: a call after a larger
    one, with f16 activations, still equals the workspace form."""
    import torch

    n_big = 16 * _cus()
    _case(q4k, 32, n_big, 12288, seed=3, x_dtype=torch.float32, reproducible=True)
    _case(q4k, 16, n_big, 2048, seed=4, x_dtype=torch.float16, reproducible=True)


def test_noalloc_refuses_beyond_its_array(q4k):
    import torch

    m, n, k = 4096, 256, 4096
    need = q4k.gemv_batched_workspace_size(m, n, k, x_dtype=torch.float16, out_dtype=torch.float32)
    assert need > q4k.NOALLOC_SCRATCH_BYTES
    w = torch.zeros(n * (k // 256) * 144, dtype=torch.uint8, device="cuda")
    x = torch.zeros((m, k), dtype=torch.float16, device="cuda")
    y = torch.full((m, n), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.gemv_batched_noalloc(w, x, y=y)
    assert ei.value.status == 2
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "a refused call launched nothing"
