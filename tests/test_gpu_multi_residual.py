"""GPU parity of the multi-matrix GEMV (q4k_gemv_multi) and the GEMV with a
residual-add epilogue (q4k_gemv_residual), through the C ABI, against the CPU
oracle on the same seeded inputs.

  * q4k_gemv_multi: every output within 2e-4 * sum_k |w_k x_k| of the oracle,
    and bitwise equal to q4k_gemv of the same matrix alone (each row is summed
    by one lane group in a fixed order, whichever launch carries it).
  * q4k_gemv_residual: every output within 2e-4 * (sum_k |w_k x_k| + |r|) of
    the oracle's f64 W x + r (the GPU adds r to its f32 sum: one more rounding,
    at most 2^-24 of that magnitude); in place (y is r) and out of place give
    the same bits.
  * q4k_gemv_multi with a gate output: the per-head de-interleave of a q
    projection's rows, bitwise the plain GEMV's values in their new places.
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


def _nan(n):
    import torch

    return torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")


def _multi_case(q4k, shapes, k, cfg, label):
    """One gemv_multi call over matrices of the given row counts; every row
    checked against the oracle and against a q4k_gemv call of its own."""
    import torch

    ws = [inputs.make_q4k(n, k, config_id=cfg, tensor_id=i) for i, n in enumerate(shapes)]
    x = inputs.make_x(1, k, config_id=cfg, tensor_id=100)[0]
    wds = [to_dev(w.reshape(-1)) for w in ws]
    xd = to_dev(x)
    ys = [_nan(n) for n in shapes]
    print(f"[case] {label}: multi rows={list(shapes)} k={k}", flush=True)
    q4k.gemv_multi(wds, xd, ys=ys, ns=list(shapes))
    torch.cuda.synchronize()
    for i, (w, n) in enumerate(zip(ws, shapes)):
        got = to_host(ys[i])
        if n == 0:
            continue
        assert np.isfinite(got).all(), f"{label}[{i}]: {int((~np.isfinite(got)).sum())} rows not written"
        yr, ar = oracle.gemv(w, x, threads=THREADS)
        _report(f"{label}[{i}] {n}x{k}", check_bound(got, yr, ar, f"{label}[{i}]"))
        alone = to_host(q4k.gemv(wds[i], xd, n=n))
        np.testing.assert_array_equal(got, alone)


# ------------------------------------------------------------------- multi
def test_multi_gdn_input_projections_0p8b(q4k):
    """qkv, z, a and b of a 0.8B linear-attention layer in one launch."""
    shapes = [inputs.SHAPES[nm][0] for nm in inputs.GDN_PROJECTIONS_0P8B]
    k = inputs.SHAPES["gdn_qkv_0p8b"][1]
    _multi_case(q4k, shapes, k, cfg=4, label="gdn 0.8b")


@pytest.mark.parametrize("shapes,k", [
    ([1], 256),
    ([3, 5], 256),
    ([7, 0, 9], 512),                        # an empty matrix in the middle
    ([1, 2, 3, 4, 5, 6, 7, 8], 768),         # eight matrices, all ragged
    ([4097, 33, 1], 1024),
    ([300, 257, 1000], 2304),
    ([129, 64, 65, 2], 4096),                # the widest rows that share a launch
    ([1025, 3], 8192),                       # wider rows: one launch per matrix
    ([17, 5], 12288),
    ([9, 2], 20480),
])
def test_multi_shapes(q4k, shapes, k):
    _multi_case(q4k, shapes, k, cfg=95, label=f"multi k={k}")


def test_multi_repeated_launches_bitwise(q4k):
    """Several calls, alternating with single-matrix calls and on two streams,
    give the same bits."""
    import torch

    k = 1024
    shapes = [6144, 2048, 16, 16]
    wds = [to_dev(inputs.make_q4k(n, k, config_id=98, tensor_id=i).reshape(-1)) for i, n in enumerate(shapes)]
    xd = to_dev(inputs.make_x(1, k, config_id=98)[0])
    base = [to_host(y) for y in q4k.gemv_multi(wds, xd, ns=shapes)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for s in (s1, s2):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                ys = q4k.gemv_multi(wds, xd, ns=shapes)
                q4k.gemv(wds[0], xd, n=shapes[0])
            s.synchronize()
            for y, b in zip(ys, base):
                np.testing.assert_array_equal(to_host(y), b)


def _split_case(q4k, shapes, split, k, cfg, label):
    """gemv_multi where matrix i (split[i] = head_dim, or 0) writes its output
    de-interleaved per head into q and gate halves: bitwise the plain GEMV's
    values reordered, and inside the oracle's bound after the oracle's own
    de-interleave."""
    import torch

    ws = [inputs.make_q4k(n, k, config_id=cfg, tensor_id=i) for i, n in enumerate(shapes)]
    x = inputs.make_x(1, k, config_id=cfg, tensor_id=100)[0]
    wds = [to_dev(w.reshape(-1)) for w in ws]
    xd = to_dev(x)
    ys = [_nan(n // 2 if hd else n) for n, hd in zip(shapes, split)]
    gs = [_nan(n // 2) if hd else None for n, hd in zip(shapes, split)]
    print(f"[case] {label}: multi rows={list(shapes)} heads={list(split)} k={k}", flush=True)
    q4k.gemv_multi(wds, xd, ys=ys, ns=list(shapes), gates=gs, head_dims=list(split))
    torch.cuda.synchronize()
    for i, (w, n, hd) in enumerate(zip(ws, shapes, split)):
        alone = to_host(q4k.gemv(wds[i], xd, n=n))
        yr, ar = oracle.gemv(w, x, threads=THREADS)
        if not hd:
            np.testing.assert_array_equal(to_host(ys[i]), alone)
            continue
        q, g = to_host(ys[i]), to_host(gs[i])
        aq, ag = oracle.split_qg(alone, hd)
        np.testing.assert_array_equal(q, aq)
        np.testing.assert_array_equal(g, ag)
        rq, rg = oracle.split_qg(yr, hd)
        sq, sg = oracle.split_qg(ar, hd)
        _report(f"{label}[{i}] q", check_bound(q, rq, sq, f"{label}[{i}] q"))
        _report(f"{label}[{i}] gate", check_bound(g, rg, sg, f"{label}[{i}] gate"))


def test_multi_split_qg_q_proj_0p8b(q4k):
    """The 0.8B q projection (8 heads x 256, q and gate interleaved per head:
    4096 x 1024) de-interleaved in the launch that also carries two other
    matrices."""
    _split_case(q4k, (4096, 512, 512), (256, 0, 0), 1024, 71, "q_proj 0.8B split")


@pytest.mark.parametrize("shapes,split,k", [
    ((24,), (4,), 256), ((2,), (1,), 512), ((64, 7), (32, 0), 2048), ((512, 256), (128, 64), 4096),
    ((8192,), (1024,), 1024), ((4,), (2,), 3072)])
def test_multi_split_qg_shapes(q4k, shapes, split, k):
    _split_case(q4k, shapes, split, k, 72, f"split {shapes}")


def test_gemv_split_qg_helper_and_k_zero(q4k):
    import torch

    n, k, hd = 1024, 2048, 64
    w = to_dev(inputs.make_q4k(n, k, config_id=73).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=73)[0])
    q, g = q4k.gemv_split_qg(w, x, hd)
    aq, ag = oracle.split_qg(to_host(q4k.gemv(w, x)), hd)
    np.testing.assert_array_equal(to_host(q), aq)
    np.testing.assert_array_equal(to_host(g), ag)
    q0 = torch.full((8,), 5.0, device="cuda")
    g0 = torch.full((8,), 5.0, device="cuda")
    q4k.gemv_split_qg(torch.empty(0, dtype=torch.uint8, device="cuda"), torch.empty(0, device="cuda"), 4, q=q0, g=g0,
                      n=16)
    assert np.all(to_host(q0) == 0) and np.all(to_host(g0) == 0)


def test_multi_k_zero_writes_zeros(q4k):
    import torch

    ys = [torch.full((n,), 5.0, device="cuda") for n in (3, 10)]
    empty_w = torch.empty(0, dtype=torch.uint8, device="cuda")
    q4k.gemv_multi([empty_w, empty_w], torch.empty(0, device="cuda"), ys=ys, ns=[3, 10])
    for y in ys:
        assert np.all(to_host(y) == 0)


# ---------------------------------------------------------------- residual
def _residual_case(q4k, n, k, cfg, label):
    import torch

    w = inputs.make_q4k(n, k, config_id=cfg, tensor_id=1)
    x = inputs.make_x(1, k, config_id=cfg, tensor_id=101)[0]
    r = inputs.make_x(1, n, config_id=cfg, tensor_id=102)[0]
    wd, xd, rd = to_dev(w.reshape(-1)), to_dev(x), to_dev(r)
    print(f"[case] {label}: residual {n}x{k}", flush=True)
    y = _nan(n)
    q4k.gemv_residual(wd, xd, rd, y=y)
    inplace = rd.clone()
    q4k.gemv_residual(wd, xd, inplace, y=inplace)
    torch.cuda.synchronize()
    got = to_host(y)
    assert np.isfinite(got).all(), f"{label}: {int((~np.isfinite(got)).sum())} rows not written"
    np.testing.assert_array_equal(to_host(inplace), got)
    np.testing.assert_array_equal(to_host(rd), r)  # r read, never written
    yr, ar = oracle.gemv_residual(w, x, r, threads=THREADS)
    _report(label, check_bound(got, yr, ar, label))
    return got


def test_residual_out_proj_0p8b(q4k):
    """Attention output projection of the 0.8B model (2048 -> 1024) plus the residual."""
    n, k = inputs.SHAPES["out_proj_0p8b"]
    _residual_case(q4k, n, k, cfg=5, label="out_proj 0.8b + r")


def test_residual_down_9b_whole(q4k):
    """The 9B FFN down projection (12288 -> 4096) plus the residual, every row
    against the oracle."""
    n, k = inputs.SHAPES["down_9b"]
    _residual_case(q4k, n, k, cfg=6, label="down 9b + r")


@pytest.mark.parametrize("n,k", [(1, 256), (7, 768), (4097, 1024), (33, 2304), (129, 8192), (65, 12288),
                                 (8195, 12288), (17, 16384), (9, 20480)])
def test_residual_shapes(q4k, n, k):
    _residual_case(q4k, n, k, cfg=7, label=f"residual {n}x{k}")


def test_residual_equals_gemv_plus_r(q4k):
    """The epilogue adds r to the same f32 sum q4k_gemv returns: y equals
    fl(gemv + r) bit for bit."""
    import torch

    for k in (1024, 4096, 12288, 20480):
        n = 513
        wd = to_dev(inputs.make_q4k(n, k, config_id=8, tensor_id=k).reshape(-1))
        xd = to_dev(inputs.make_x(1, k, config_id=8, tensor_id=k)[0])
        rd = to_dev(inputs.make_x(1, n, config_id=8, tensor_id=k + 1)[0])
        plain = q4k.gemv(wd, xd)
        fused = q4k.gemv_residual(wd, xd, rd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(fused), to_host(plain + rd))


def test_residual_k_zero_copies_r(q4k):
    import torch

    r = torch.arange(10, dtype=torch.float32, device="cuda")
    y = torch.full((10,), 5.0, device="cuda")
    empty_w = torch.empty(0, dtype=torch.uint8, device="cuda")
    q4k.gemv_residual(empty_w, torch.empty(0, device="cuda"), r, y=y, n=10)
    np.testing.assert_array_equal(to_host(y), np.arange(10, dtype=np.float32))
    q4k.gemv_residual(empty_w, torch.empty(0, device="cuda"), r, y=r, n=10)
    np.testing.assert_array_equal(to_host(r), np.arange(10, dtype=np.float32))
