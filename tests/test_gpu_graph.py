"""HIP graph capture of the decode calls: a graph holding a fused SwiGLU, a
K-split GEMV with a residual, a multi-matrix GEMV, a batch-1 GEMV and a Q8_0
GEMV, replayed several times with the program's own eager work and
synchronizations between replays; every replay must equal the eager results
bit for bit (no call on this path records a memset or allocates)."""

from __future__ import annotations

import numpy as np
import pytest

from gpu_helpers import to_dev
from q4_dequant_gemv_amd import inputs

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_equal_eager():
    import torch

    from q4_dequant_gemv_amd import q4k

    torch.cuda.init()
    k, nff, nv = 2048, 6144, 5000
    wg = to_dev(inputs.make_q4k(nff, k, config_id=80, tensor_id=0).reshape(-1))
    wu = to_dev(inputs.make_q4k(nff, k, config_id=80, tensor_id=1).reshape(-1))
    wd = to_dev(inputs.make_q4k(k, nff, config_id=80, tensor_id=2).reshape(-1))
    wq = [to_dev(inputs.make_q4k(n, k, config_id=80, tensor_id=3 + i).reshape(-1)) for i, n in enumerate((512, 64, 3))]
    wl = to_dev(inputs.make_q4k(nv, k, config_id=80, tensor_id=6).reshape(-1))
    w8 = to_dev(inputs.make_q8_0(777, k, config_id=80, tensor_id=7).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=80)[0])
    r = to_dev(inputs.make_x(1, k, config_id=80, tensor_id=101)[0])
    h = torch.empty(nff, device="cuda")
    y = torch.empty(k, device="cuda")
    qs = [torch.empty(n, device="cuda") for n in (512, 64, 3)]
    lg = torch.empty(nv, device="cuda")
    y8 = torch.empty(777, device="cuda")

    def step():
        q4k.fused_swiglu(wg, wu, x, h=h)
        q4k.gemv_residual(wd, h, r, y=y)
        q4k.gemv_multi(wq, y, ys=qs, ns=[512, 64, 3])
        q4k.gemv(wl, y, y=lg)
        q4k.q8_0_gemv(w8, y, y=y8)

    outs = (h, y, *qs, lg, y8)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, ref)):
            assert torch.equal(t, e), f"replay {rep}: output {i} differs from the eager run"
        step()  # the program's own eager work between replays
        torch.cuda.synchronize()
        assert np.isfinite(lg.cpu().numpy()).all()


def test_full_size_9b_step_in_a_graph():
    """The decode step at its full 9B sizes, in the launch configuration the
    benchmark times (a HIP graph of whole steps): fused gate+up SwiGLU
    (2 x 12288 x 4096), down (4096 x 12288), lm_head (248320 x 4096).
    Replays equal the eager step bit for bit; each stage is checked against
    the oracle on the GPU's own input to that stage (h, y), every output."""
    import torch

    import oracle
    from gpu_helpers import THREADS, check_bound, check_swiglu_bound, to_host
    from q4_dequant_gemv_amd import q4k

    torch.cuda.init()
    oracle.build(force=False)
    nff, k = inputs.SHAPES["gate_9b"]
    nv = inputs.SHAPES["lm_head_9b"][0]
    print("[case] full-size 9B step in a graph", flush=True)
    wg_h = inputs.make_q4k(nff, k, config_id=2, tensor_id=0)
    wu_h = inputs.make_q4k(nff, k, config_id=2, tensor_id=1)
    wd_h = inputs.make_q4k(k, nff, config_id=2, tensor_id=2)
    wl_h = inputs.make_q4k(nv, k, config_id=3, tensor_id=0)
    x_h = inputs.make_x(1, k, config_id=2)[0]
    wg, wu, wd, wl = (to_dev(a.reshape(-1)) for a in (wg_h, wu_h, wd_h, wl_h))
    x = to_dev(x_h)
    h = torch.empty(nff, device="cuda")
    y = torch.empty(k, device="cuda")
    logits = torch.empty(nv, device="cuda")

    def step():
        q4k.fused_swiglu(wg, wu, x, h=h)
        q4k.gemv(wd, h, y=y)
        q4k.gemv(wl, y, y=logits)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (h, y, logits)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(3):
            step()
    for rep in range(3):
        for t in (h, y, logits):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for t, e, nm in zip((h, y, logits), ref, ("h", "y", "logits")):
            assert torch.equal(t, e), f"replay {rep}: {nm} differs from the eager step"
        step()
        torch.cuda.synchronize()
    hh, yy, lg = (to_host(t) for t in ref)
    sw = oracle.fused_swiglu(wg_h, wu_h, x_h, threads=THREADS)
    check_swiglu_bound(hh, sw, "9B step: SwiGLU")
    yr, ar = oracle.gemv(wd_h, hh, threads=THREADS)
    check_bound(yy, yr, ar, "9B step: down")
    lr, la = oracle.gemv(wl_h, yy, threads=THREADS)
    check_bound(lg, lr, la, "9B step: lm_head")
