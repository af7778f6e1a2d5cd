"""The caller-workspace forms of the batched and prefill calls
(q4k_gemv_batched_ws, q4k_prefill_gemm_ws) through the C ABI.

  * With a workspace of the queried size they compute exactly what the
    allocating calls compute: bit for bit where each output is summed by one
    workgroup in a fixed order (every prefill shape; batched shapes with at
    least 16 rows per compute unit), and within the oracle's bound where the
    batched call splits K across workgroups and adds with atomics.
  * A workspace that is too small, misaligned or overlapping an operand is
    refused before anything runs; a larger one, or one placed at an offset in
    a bigger buffer, works the same.
  * Recorded into a HIP graph (no allocation node, no memset), replays equal
    the eager results bit for bit, with the program's own eager work and
    synchronisations between replays.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import THREADS, batched_on_gemv_kernels, check_bound, check_bound_f16, to_dev, to_host
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


def _workspace(nbytes, offset=0):
    """A uint8 device buffer of nbytes starting `offset` bytes into a larger,
    256-byte aligned allocation (None for 0 bytes)."""
    import torch

    if nbytes == 0:
        return None
    base = torch.empty(nbytes + offset + 256, dtype=torch.uint8, device="cuda")
    skip = (-base.data_ptr()) % 256 + offset
    ws = base[skip:skip + nbytes]
    assert ws.data_ptr() % 256 == 0 or offset % 256 != 0
    return ws


@pytest.mark.parametrize("m,n,k", [(2, 4096, 2048), (16, 8192, 1024), (64, 4100, 2048), (100, 4096, 2304),
                                   (33, 513, 1024), (4, 70, 12288), (17, 300, 4096), (3, 1000, 4096),
                                   (5, 4096, 1024), (4, 20000, 1024)])
@pytest.mark.parametrize("xd,yd", [("f32", "f32"), ("f16", "f16"), ("f16", "f32")])
def test_batched_ws_matches_allocating_call(q4k, m, n, k, xd, yd):
    import torch

    dt = {"f32": torch.float32, "f16": torch.float16}
    print(f"[case] batched_ws m={m} {n}x{k} {xd}->{yd}", flush=True)
    w = inputs.make_q4k(n, k, config_id=90, tensor_id=k)
    x = inputs.make_x(m, k, config_id=90, tensor_id=m)
    if xd == "f16":
        x = x.astype(np.float16)
    wd, xt = to_dev(w.reshape(-1)), to_dev(x)
    need = q4k.gemv_batched_workspace_size(m, n, k, x_dtype=dt[xd], out_dtype=dt[yd])
    # a few tokens run on the streaming GEMV kernels, which need none
    small = batched_on_gemv_kernels(m, n, k)
    assert (need == 0) == small
    y_ws = q4k.gemv_batched_ws(wd, xt, None if small else _workspace(need), out_dtype=dt[yd])
    y_al = q4k.gemv_batched_dt(wd, xt, out_dtype=dt[yd])
    torch.cuda.synchronize()
    split = not small and n < 16 * _cus() and k >= 512
    if not split:
        assert torch.equal(y_ws, y_al), "workspace form differs from the allocating call"
        # a bigger workspace at an odd multiple of 256 bytes into a buffer: same bits
        y2 = q4k.gemv_batched_ws(wd, xt, _workspace(need + 4096, offset=768), out_dtype=dt[yd])
        assert torch.equal(y2, y_al)
    yr, ar = oracle.gemv_batched(w, x.astype(np.float32), threads=THREADS)
    got = to_host(y_ws.float())
    if yd == "f32":
        check_bound(got, yr, ar, f"batched_ws m={m} {n}x{k}")
    else:
        check_bound_f16(got, yr, ar, f"batched_ws m={m} {n}x{k} f16")


def test_batched_ws_needs_no_workspace_for_one_token(q4k):
    import torch

    n, k = 1000, 2048
    w = to_dev(inputs.make_q4k(n, k, config_id=91).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=91))
    assert q4k.gemv_batched_workspace_size(1, n, k) == 0
    y = q4k.gemv_batched_ws(w, x, None)
    assert torch.equal(y, q4k.gemv_batched(w, x))


def test_batched_ws_rejects_bad_workspaces(q4k):
    import torch

    m, n, k = 8, 4096, 1024
    w = to_dev(inputs.make_q4k(n, k, config_id=92).reshape(-1))
    x = to_dev(inputs.make_x(m, k, config_id=92))
    need = q4k.gemv_batched_workspace_size(m, n, k)
    y = torch.full((m, n), 7.0, device="cuda")
    for bad in (None, _workspace(need - 256), _workspace(need, offset=16)):
        with pytest.raises(q4k.Q4KError) as ei:
            q4k.gemv_batched_ws(w, x, bad, y=y)
        assert ei.value.status in (1, 3)
    # a workspace that overlaps the output
    big = torch.empty(need + m * n * 4 + 256, dtype=torch.uint8, device="cuda")
    skip = (-big.data_ptr()) % 256
    yv = big[skip:skip + m * n * 4].view(torch.float32).view(m, n)
    with pytest.raises(q4k.Q4KError) as ei:
        q4k.gemv_batched_ws(w, x, big[skip:skip + need], y=yv)
    assert ei.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(y == 7.0), "a refused call wrote its output"


@pytest.mark.parametrize("m,n,k", [(128, 1024, 2048), (300, 700, 4096), (256, 4096, 4096), (1, 64, 1024),
                                   (129, 96, 12288)])
@pytest.mark.parametrize("yd", ["f32", "f16"])
def test_prefill_ws_matches_allocating_call(q4k, m, n, k, yd):
    import torch

    dt = {"f32": torch.float32, "f16": torch.float16}
    print(f"[case] prefill_ws m={m} {n}x{k} {yd}", flush=True)
    w = inputs.make_q4k(n, k, config_id=93, tensor_id=k)
    x = inputs.make_x(m, k, config_id=93, tensor_id=m).astype(np.float16)
    wd, xt = to_dev(w.reshape(-1)), to_dev(x)
    need = q4k.prefill_workspace_size(m, n, k, out_dtype=dt[yd])
    assert need >= 2 * 128 * k
    y_ws = q4k.prefill_gemm_ws(wd, xt, _workspace(need), out_dtype=dt[yd])
    y_al = q4k.prefill_gemm(wd, xt, out_dtype=dt[yd])
    torch.cuda.synchronize()
    assert torch.equal(y_ws, y_al), "workspace form differs from the allocating call"
    with pytest.raises(q4k.Q4KError):
        q4k.prefill_gemm_ws(wd, xt, _workspace(need - 256), out_dtype=dt[yd])
    if m * n <= 300 * 1024:
        yr, ar = oracle.gemv_batched(w, x.astype(np.float32), threads=THREADS)
        got = to_host(y_ws.float())
        if yd == "f32":
            check_bound(got, yr, ar, f"prefill_ws m={m} {n}x{k}")
        else:
            check_bound_f16(got, yr, ar, f"prefill_ws m={m} {n}x{k} f16")


def test_workspace_calls_in_a_graph_replay_equal_eager(q4k):
    import torch

    cus = _cus()
    k = 2048
    nb = 16 * cus           # one fixed-order sum per output: bitwise reproducible
    wb = to_dev(inputs.make_q4k(nb, k, config_id=94, tensor_id=0).reshape(-1))
    wp = to_dev(inputs.make_q4k(512, k, config_id=94, tensor_id=1).reshape(-1))  # prefill with K split
    xb = to_dev(inputs.make_x(24, k, config_id=94).astype(np.float16))
    xp = to_dev(inputs.make_x(200, k, config_id=94, tensor_id=2).astype(np.float16))
    ws_b = _workspace(q4k.gemv_batched_workspace_size(24, nb, k, x_dtype=torch.float16, out_dtype=torch.float16))
    ws_p = _workspace(q4k.prefill_workspace_size(200, 512, k))
    yb = torch.empty((24, nb), dtype=torch.float16, device="cuda")
    yp = torch.empty((200, 512), dtype=torch.float32, device="cuda")
    # two tokens (the streaming GEMV, no workspace) and sixteen (the streamed
    # matrix-core kernel) over the same rows
    x2 = to_dev(inputs.make_x(2, k, config_id=94, tensor_id=3))
    x16 = to_dev(inputs.make_x(16, k, config_id=94, tensor_id=4))
    assert batched_on_gemv_kernels(2, nb, k) and not batched_on_gemv_kernels(16, nb, k)
    assert q4k.gemv_batched_workspace_size(2, nb, k) == 0
    ws_16 = _workspace(q4k.gemv_batched_workspace_size(16, nb, k))
    y2 = torch.empty((2, nb), dtype=torch.float32, device="cuda")
    y16 = torch.empty((16, nb), dtype=torch.float32, device="cuda")

    def step():
        q4k.gemv_batched_ws(wb, xb, ws_b, y=yb)
        q4k.prefill_gemm_ws(wp, xp, ws_p, y=yp)
        q4k.gemv_batched_ws(wb, x2, None, y=y2)
        q4k.gemv_batched_ws(wb, x16, ws_16, y=y16)

    step()
    torch.cuda.synchronize()
    ref = [yb.clone(), yp.clone(), y2.clone(), y16.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (yb, yp, y2, y16):
            t.fill_(float("nan"))
        ws_b.fill_(0xAB)
        ws_p.fill_(0xCD)      # stale workspace contents must not matter
        ws_16.fill_(0xEF)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yb, ref[0]), f"replay {rep}: batched output differs"
        assert torch.equal(yp, ref[1]), f"replay {rep}: prefill output differs"
        assert torch.equal(y2, ref[2]), f"replay {rep}: two-token output differs"
        assert torch.equal(y16, ref[3]), f"replay {rep}: sixteen-token output differs"
        step()
        torch.cuda.synchronize()


def test_plain_calls_reuse_per_stream_scratch(q4k):
    """The calls made without a workspace keep one scratch buffer per stream:
    calls alternating between two streams that run at the same time, a call
    that needs more scratch than the stream's buffer holds (it grows) and a
    smaller one after it all give the bits of the workspace form; a plain call
    recorded into a HIP graph (which allocates for itself there) replays to
    the eager result."""
    import torch

    cus = _cus()
    k = 2048
    nb = 16 * cus
    print(f"[case] per-stream scratch n={nb} k={k}", flush=True)
    w = to_dev(inputs.make_q4k(nb, k, config_id=93, tensor_id=7).reshape(-1))
    xs = [to_dev(inputs.make_x(m, k, config_id=93, tensor_id=10 + i)) for i, m in enumerate((16, 40, 16, 64))]

    def ref(x):
        y = torch.empty((x.shape[0], nb), dtype=torch.float32, device="cuda")
        ws = _workspace(q4k.gemv_batched_workspace_size(x.shape[0], nb, k))
        q4k.gemv_batched_ws(w, x, ws, y=y)
        torch.cuda.synchronize()
        return y

    refs = [ref(x) for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    outs = []
    for rnd in range(6):
        for si, st in enumerate(streams):
            i = (rnd + si) % len(xs)   # each stream walks the sizes: 16, 40 (grows), 16, 64 (grows), ...
            y = torch.full((xs[i].shape[0], nb), float("nan"), dtype=torch.float32, device="cuda")
            with torch.cuda.stream(st):
                q4k.gemv_batched(w, xs[i], y=y)
            outs.append((i, y))
    for st in streams:
        torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for i, y in outs:
        assert torch.equal(y, refs[i]), f"plain call on size {xs[i].shape[0]} differs from the workspace form"
    # a plain call inside a graph
    yg = torch.empty((16, nb), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q4k.gemv_batched(w, xs[0], y=yg)
    for rep in range(3):
        yg.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yg, refs[0]), f"replay {rep} of a plain call differs"
        q4k.gemv_batched(w, xs[2], y=torch.empty_like(yg))   # eager work between replays
        torch.cuda.synchronize()
