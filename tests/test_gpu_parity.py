"""GPU parity: every entry point of libq4k.so (called through the C ABI via
the thin binding) against the CPU oracle on the same seeded inputs.

  * q4k_dequant: bitwise equal to the oracle's f32 dequant.
  * q4k_gemv / q4k_gemv_batched: every output within 2e-4 * sum_k |w_k x_k|.
  * q4k_fused_swiglu: within the bound derived from the GEMV bound.

Every output is compared: small shapes and the full-size matrices of the
Qwen3.5 shapes (issue #3346) alike, the latter run on the GPU in the same
launch configuration the benchmark times, with the oracle's rows split over
host threads.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import THREADS, batched_on_gemv_kernels, check_bound, check_swiglu_bound, to_dev, to_host
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


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("n,k", [(1024, 1024), (4096, 1024), (1024, 2048), (37, 256), (3, 12288), (5, 20480)])
def test_dequant_bit_exact(q4k, n, k):
    w = inputs.make_q4k(n, k, config_id=90, tensor_id=k)
    got = to_host(q4k.dequant(to_dev(w), k))
    want = oracle.dequant(w, k, threads=THREADS)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


def test_dequant_every_f16_pattern(q4k):
    """d and dmin take all 65,536 binary16 patterns (subnormals, inf, NaN)."""
    nb = 65536
    g = np.random.default_rng(21)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    sc = g.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    bits = np.arange(nb, dtype=np.uint32).astype(np.uint16)
    w = inputs.assemble_blocks(qs, sc, bits.view(np.float16), np.roll(bits, 12345).view(np.float16))
    got = to_host(q4k.dequant(to_dev(w.reshape(-1)), 256))
    want = oracle.dequant(w.reshape(-1), 256, threads=THREADS)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_dequant_row_chunks_of_lm_head_0p8b(q4k):
    """Rows of the 0.8B lm_head (248320 x 1024) through pointer offsets."""
    import torch

    n, k = inputs.SHAPES["lm_head_0p8b"]
    w = inputs.make_q4k(n, k, config_id=1, tensor_id=3)
    wd = to_dev(w.reshape(-1))
    rb = inputs.row_bytes(k)
    for r0, cnt in ((0, 512), (123_457, 300), (n - 777, 777)):
        out = torch.empty((cnt, k), dtype=torch.float32, device="cuda")
        q4k.dequant(wd[r0 * rb:(r0 + cnt) * rb], k, out=out)
        want = oracle.dequant(w[r0:r0 + cnt], k, threads=THREADS)
        np.testing.assert_array_equal(to_host(out).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("name,tid", [("gate_9b", 0), ("down_9b", 2)])
def test_dequant_9b_ffn_whole(q4k, name, tid):
    """The 9B FFN matrices (28.3 MB of Q4_K, 201 MB of f32) whole, bit for bit."""
    import torch

    n, k = inputs.SHAPES[name]
    w = inputs.make_q4k(n, k, config_id=2, tensor_id=tid)
    out = torch.empty((n, k), dtype=torch.float32, device="cuda")
    q4k.dequant(to_dev(w.reshape(-1)), k, out=out)
    want = oracle.dequant(w, k, threads=THREADS)
    np.testing.assert_array_equal(to_host(out).view(np.uint32), want.view(np.uint32))


def test_dequant_lm_head_0p8b_whole(q4k):
    """The whole 0.8B lm_head (248320 x 1024: 1 GB of f32, written with
    non-temporal stores, the path for outputs of 256 MiB or more) bit for bit;
    and both sides of that switch (65535 and 65536 rows of 1024 weights:
    256 MiB less 4 KiB, and exactly 256 MiB of output)."""
    import torch

    n, k = inputs.SHAPES["lm_head_0p8b"]
    w = inputs.make_q4k(n, k, config_id=1, tensor_id=3)
    wd = to_dev(w.reshape(-1))
    out = torch.full((n, k), float("nan"), dtype=torch.float32, device="cuda")
    q4k.dequant(wd, k, out=out)
    want = oracle.dequant(w, k, threads=THREADS)
    np.testing.assert_array_equal(to_host(out).view(np.uint32), want.view(np.uint32))
    del out
    rb = inputs.row_bytes(k)
    for cnt in (65535, 65536):
        o = torch.full((cnt, k), float("nan"), dtype=torch.float32, device="cuda")
        q4k.dequant(wd[:cnt * rb], k, out=o)
        np.testing.assert_array_equal(to_host(o).view(np.uint32), want[:cnt].view(np.uint32))


def test_dequant_row_chunks_of_lm_head_9b(q4k):
    """Rows of the 9B lm_head (248320 x 4096, 572 MB) through pointer offsets:
    the first rows, a middle range and the last rows."""
    import torch

    n, k = inputs.SHAPES["lm_head_9b"]
    w = inputs.make_q4k(n, k, config_id=3, tensor_id=0)
    wd = to_dev(w.reshape(-1))
    rb = inputs.row_bytes(k)
    for r0, cnt in ((0, 1024), (131_071, 2049), (n - 1000, 1000)):
        out = torch.empty((cnt, k), dtype=torch.float32, device="cuda")
        q4k.dequant(wd[r0 * rb:(r0 + cnt) * rb], k, out=out)
        want = oracle.dequant(w[r0:r0 + cnt], k, threads=THREADS)
        np.testing.assert_array_equal(to_host(out).view(np.uint32), want.view(np.uint32))


# --------------------------------------------------------------------- gemv
def _gemv_case(q4k, w, x):
    y = to_host(q4k.gemv(to_dev(w.reshape(-1)), to_dev(x)))
    yr, ar = oracle.gemv(w, x, threads=THREADS)
    return y, yr, ar


def test_gemv_square_1k(q4k):
    """1024 x 1024, seed 0: the small case, compared whole."""
    n, k = inputs.SHAPES["square_1k"]
    w = inputs.make_q4k(n, k, config_id=0, tensor_id=0)
    x = inputs.make_x(1, k, config_id=0)[0]
    _report("square_1k", check_bound(*_gemv_case(q4k, w, x), "square_1k"))


@pytest.mark.parametrize("name,tid", [("q_proj_0p8b", 1), ("out_proj_0p8b", 2)])
def test_gemv_0p8b_projections(q4k, name, tid):
    n, k = inputs.SHAPES[name]
    w = inputs.make_q4k(n, k, config_id=1, tensor_id=tid)
    x = inputs.make_x(1, k, config_id=1, tensor_id=100 + tid)[0]
    _report(name, check_bound(*_gemv_case(q4k, w, x), name))


@pytest.mark.parametrize("name,cfg,tid", [("lm_head_0p8b", 1, 3), ("lm_head_9b", 3, 0), ("down_9b", 2, 2)])
def test_gemv_full_size_whole(q4k, name, cfg, tid):
    """Whole matrix on the GPU (y pre-filled with NaN, so a row that no wave
    wrote shows up), every row against the oracle."""
    import torch

    n, k = inputs.SHAPES[name]
    w = inputs.make_q4k(n, k, config_id=cfg, tensor_id=tid)
    x = inputs.make_x(1, k, config_id=cfg, tensor_id=100 + tid)[0]
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    q4k.gemv(to_dev(w.reshape(-1)), to_dev(x), y=y)
    got = to_host(y)
    assert np.isfinite(got).all(), f"{int((~np.isfinite(got)).sum())} rows not written"
    yr, ar = oracle.gemv(w, x, threads=THREADS)
    _report(name, check_bound(got, yr, ar, name))


def test_gemv_concurrent_streams_bitwise(q4k):
    """Repeated launches on one stream, and launches on two streams running
    at the same time, all write every row with the same bits: rows are
    assigned to waves statically and each row is summed by one wave in a
    fixed order, so nothing depends on timing or on another launch."""
    import torch

    n, k = inputs.SHAPES["lm_head_0p8b"]
    w = to_dev(inputs.make_q4k(n, k, config_id=97, tensor_id=0).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=97)[0])
    base = to_host(q4k.gemv(w, x))
    assert np.isfinite(base).all()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        for s in (s1, s2):
            y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                q4k.gemv(w, x, y=y)
            outs.append(y)
    torch.cuda.synchronize()
    for _ in range(3):
        outs.append(q4k.gemv(w, x))
    for y in outs:
        np.testing.assert_array_equal(to_host(y), base)
    h0 = None
    for s in (None, s1, s2, s1):
        h = torch.full((12288,), float("nan"), dtype=torch.float32, device="cuda")
        wg = to_dev(inputs.make_q4k(12288, 4096, config_id=97, tensor_id=1).reshape(-1)) if h0 is None else wg
        wu = to_dev(inputs.make_q4k(12288, 4096, config_id=97, tensor_id=2).reshape(-1)) if h0 is None else wu
        x2 = to_dev(inputs.make_x(1, 4096, config_id=97, tensor_id=3)[0]) if h0 is None else x2
        if s is None:
            q4k.fused_swiglu(wg, wu, x2, h=h)
        else:
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                q4k.fused_swiglu(wg, wu, x2, h=h)
        torch.cuda.synchronize()
        got = to_host(h)
        if h0 is None:
            assert np.isfinite(got).all()
            h0 = got
        np.testing.assert_array_equal(got, h0)


@pytest.mark.parametrize("n,k", [(1, 256), (3, 256), (5, 512), (7, 768), (4097, 1024), (33, 2304), (129, 8192),
                                 (65, 12288), (17, 16384), (9, 20480), (300, 3072)])
def test_gemv_edge_shapes(q4k, n, k):
    w = inputs.make_q4k(n, k, config_id=91, tensor_id=k)
    x = inputs.make_x(1, k, config_id=91, tensor_id=k)[0]
    _report(f"gemv {n}x{k}", check_bound(*_gemv_case(q4k, w, x), f"gemv {n}x{k}"))


@pytest.mark.parametrize("n,k", [(20483, 12288), (16389, 8192), (9001, 16384)])
def test_gemv_split_rows_many_iterations(q4k, n, k):
    """Rows wider than 4096 are split over several waves whose partial sums
    meet in LDS; these sizes give every workgroup more block iterations than
    one exchange holds, and a ragged last iteration.  Two runs agree bitwise
    (the partials are added in a fixed order)."""
    import torch

    w = inputs.make_q4k(n, k, config_id=96, tensor_id=k)
    x = inputs.make_x(1, k, config_id=96, tensor_id=k)[0]
    wd, xd = to_dev(w.reshape(-1)), to_dev(x)
    y1 = q4k.gemv(wd, xd)
    y2 = q4k.gemv(wd, xd)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y, a = oracle.gemv(w, x, threads=THREADS)
    _report(f"gemv split {n}x{k}", check_bound(to_host(y1), y, a, f"gemv split {n}x{k}"))


def test_gemv_row_subrange_matches_whole(q4k):
    """A row range passed by pointer offsets gives the same bits as the whole call."""
    import torch

    n, k = 1000, 4096
    w = inputs.make_q4k(n, k, config_id=92, tensor_id=0)
    x = to_dev(inputs.make_x(1, k, config_id=92)[0])
    wd = to_dev(w.reshape(-1))
    full = to_host(q4k.gemv(wd, x))
    rb = inputs.row_bytes(k)
    part = torch.empty(300, dtype=torch.float32, device="cuda")
    q4k.gemv(wd[517 * rb:817 * rb], x, y=part)
    np.testing.assert_array_equal(to_host(part), full[517:817])


def test_eight_way_shards_of_the_9b_decode_matrices(q4k):
    """One GPU's share of an eight-way split, at its real shapes:
    * lm_head and gate/up by rows (pointer offsets): each shard's outputs are
      the whole call's rows, bit for bit (31,040 and 1536 rows);
    * down by K: each GPU holds its 1536 columns (6 super-blocks of every row)
      as a matrix of its own and produces a partial y; the eight partials,
      summed as an all-reduce would, are inside the whole product's bound."""
    import torch

    print("[case] eight-way shards", flush=True)
    g = 8
    # lm_head 9B: rows
    n, k = inputs.SHAPES["lm_head_9b"]
    ns = inputs.SHAPES["lm_head_9b_shard8"][0]
    assert ns * g == n
    wl = to_dev(inputs.make_q4k(n, k, config_id=3, tensor_id=0).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=3)[0])
    full = q4k.gemv(wl, x)
    rb = inputs.row_bytes(k)
    for s in (0, 3, 7):
        part = q4k.gemv(wl[s * ns * rb:(s + 1) * ns * rb], x)
        assert torch.equal(part, full[s * ns:(s + 1) * ns]), f"lm_head shard {s}"
    del wl, full
    # gate/up 9B: rows, through the fused SwiGLU
    n, k = inputs.SHAPES["gate_9b"]
    ns = inputs.SHAPES["gate_9b_shard8"][0]
    wg = to_dev(inputs.make_q4k(n, k, config_id=2, tensor_id=0).reshape(-1))
    wu = to_dev(inputs.make_q4k(n, k, config_id=2, tensor_id=1).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=2)[0])
    full = q4k.fused_swiglu(wg, wu, x)
    rb = inputs.row_bytes(k)
    for s in range(g):
        sl = slice(s * ns * rb, (s + 1) * ns * rb)
        assert torch.equal(q4k.fused_swiglu(wg[sl], wu[sl], x), full[s * ns:(s + 1) * ns]), f"gate/up shard {s}"
    del wg, wu, full
    # down 9B: split K
    n, k = inputs.SHAPES["down_9b"]
    ks = inputs.SHAPES["down_9b_kshard8"][1]
    assert ks * g == k
    w = inputs.make_q4k(n, k, config_id=2, tensor_id=2)
    xh = inputs.make_x(1, k, config_id=2, tensor_id=5)[0]
    sb = ks // 256
    w_rows = w.reshape(n, -1)
    acc = np.zeros(n, dtype=np.float64)
    for s in range(g):
        shard = np.ascontiguousarray(w_rows[:, s * sb * 144:(s + 1) * sb * 144])
        ys = q4k.gemv(to_dev(shard.reshape(-1)), to_dev(np.ascontiguousarray(xh[s * ks:(s + 1) * ks])))
        acc += to_host(ys).astype(np.float64)
    yr, ar = oracle.gemv(w, xh, threads=THREADS)
    _report("down split-K 8 ways", check_bound(acc, yr, ar, "down split-K sum"))


def test_gemv_special_values(q4k):
    n, k = 64, 1024
    x = inputs.make_x(1, k, config_id=93)[0]
    # all-zero nibbles: every weight is -dmin*m
    w = inputs.make_q4k(n, k, config_id=93, tensor_id=1).reshape(-1, 144)
    w[:, 16:] = 0
    _report("zero codes", check_bound(*_gemv_case(q4k, w.reshape(n, -1), x), "zero codes"))
    # x == 0 gives exactly 0
    w = inputs.make_q4k(n, k, config_id=93, tensor_id=2)
    y = to_host(q4k.gemv(to_dev(w.reshape(-1)), to_dev(np.zeros(k, np.float32))))
    assert np.all(y == 0)
    # every weight exactly zero through cancellation: q = 1, sc = m, d = dmin
    blocks = inputs.make_q4k(n, k, config_id=93, tensor_id=3).reshape(-1, 144).copy()
    blocks[:, 16:] = 0x11
    blocks[:, 2:4] = blocks[:, 0:2]
    from independent_decoder import pack_scales

    rng = np.random.default_rng(5)
    for b in blocks:
        v = list(rng.integers(1, 64, 8))
        b[4:16] = np.frombuffer(pack_scales(v, v), np.uint8)
    assert np.all(oracle.dequant(blocks.reshape(-1), k) == 0)
    y = to_host(q4k.gemv(to_dev(blocks.reshape(-1)), to_dev(x)))
    assert np.all(y == 0)
    # partial cancellation: a few sub-blocks cancel, the rest do not
    blocks = inputs.make_q4k(n, k, config_id=93, tensor_id=4).reshape(-1, 144).copy()
    blocks[::3, 16:48] = 0x11
    _report("partial cancel", check_bound(*_gemv_case(q4k, blocks.reshape(n, -1), x), "partial cancel"))
    # activations spanning 16 binades (outlier channels), and tiny / huge scales
    xs = (x * np.exp2(np.random.default_rng(6).integers(-8, 9, k))).astype(np.float32)
    _report("wide x", check_bound(*_gemv_case(q4k, w, xs), "wide x"))
    for s in (1e-30, 1e25):
        xs = (x * np.float32(s)).astype(np.float32)
        _report(f"x*{s}", check_bound(*_gemv_case(q4k, w, xs), f"x*{s}"))
    # weights with arbitrary finite f16 d, dmin (subnormals included)
    wb = inputs.make_q4k(n, k, config_id=93, tensor_id=5).reshape(-1, 144).copy()
    bits = np.random.default_rng(7).integers(0, 0x7800, size=(wb.shape[0], 2), dtype=np.uint16)
    wb[:, 0:4] = bits.view(np.uint8).reshape(-1, 4)
    _report("f16 range", check_bound(*_gemv_case(q4k, wb.reshape(n, -1), x), "f16 range"))
    # a non-finite activation poisons every output (each row reads all of x)
    xn = x.copy()
    xn[77] = np.nan
    y = to_host(q4k.gemv(to_dev(w.reshape(-1)), to_dev(xn)))
    assert np.all(np.isnan(y))


def test_gemv_k_zero_writes_zeros(q4k):
    import torch

    y = torch.full((10,), 5.0, device="cuda")
    q4k.gemv(torch.empty(0, dtype=torch.uint8, device="cuda"), torch.empty(0, device="cuda"), y=y, n=10)
    assert np.all(to_host(y) == 0)


def test_gemv_on_side_stream_and_deterministic(q4k):
    import torch

    n, k = 2048, 4096
    w = to_dev(inputs.make_q4k(n, k, config_id=94, tensor_id=0).reshape(-1))
    x = to_dev(inputs.make_x(1, k, config_id=94)[0])
    base = to_host(q4k.gemv(w, x))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        again = q4k.gemv(w, x)
    s.synchronize()
    np.testing.assert_array_equal(to_host(again), base)
    for _ in range(3):
        np.testing.assert_array_equal(to_host(q4k.gemv(w, x)), base)


# ------------------------------------------------------------------- swiglu
def test_swiglu_ffn_9b(q4k):
    """Gate and up of the 9B FFN (12288 x 4096 each), every output against
    the oracle."""
    n, k = inputs.SHAPES["gate_9b"]
    wg = inputs.make_q4k(n, k, config_id=2, tensor_id=0)
    wu = inputs.make_q4k(n, k, config_id=2, tensor_id=1)
    x = inputs.make_x(1, k, config_id=2, tensor_id=100)[0]
    h = to_host(q4k.fused_swiglu(to_dev(wg.reshape(-1)), to_dev(wu.reshape(-1)), to_dev(x)))
    ref = oracle.fused_swiglu(wg, wu, x, threads=THREADS)
    _report("swiglu 9b", check_swiglu_bound(h, ref, "swiglu 9b"))


@pytest.mark.parametrize("n,k", [(1, 256), (77, 1024), (300, 2048), (65, 12288), (9, 16384), (8195, 12288),
                                 (4103, 8192), (2049, 16384)])
def test_swiglu_shapes(q4k, n, k):
    wg = inputs.make_q4k(n, k, config_id=95, tensor_id=2 * k)
    wu = inputs.make_q4k(n, k, config_id=95, tensor_id=2 * k + 1)
    x = inputs.make_x(1, k, config_id=95, tensor_id=k)[0]
    h = to_host(q4k.fused_swiglu(to_dev(wg.reshape(-1)), to_dev(wu.reshape(-1)), to_dev(x)))
    ref = oracle.fused_swiglu(wg, wu, x, threads=THREADS)
    _report(f"swiglu {n}x{k}", check_swiglu_bound(h, ref, f"swiglu {n}x{k}"))


# ------------------------------------------------------------------ batched
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100])
def test_batched_small(q4k, m):
    n, k = 200, 2048
    w = inputs.make_q4k(n, k, config_id=96, tensor_id=0)
    xs = inputs.make_x(m, k, config_id=96, tensor_id=m)
    y = to_host(q4k.gemv_batched(to_dev(w.reshape(-1)), to_dev(xs)))
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    _report(f"batched m={m}", check_bound(y, yr, ar, f"batched m={m} {n}x{k}"))


def _random_batched_cases(count=24, seed=2024):
    """Seeded (m, rows, k) draws over the batched call's whole range: m from 2
    to 80, k from 256 to 16384 and 1 to 6000 rows; and, alternately, rows a
    multiple (1, 2, 3 or 8) of 16 * CUs give or take 16 (the kernel-choice
    switches, scaled by the CU count at run time) at k = 1024, 4096, 4352 or
    12288; at most about 1.6e9 multiply-adds each (on 256 CUs)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        if len(out) % 2 == 0:
            m = int(rng.integers(2, 81))
            k = 256 * int(rng.integers(1, 65))
            rows = ("free", int(rng.integers(1, 6001)))
            n_est = rows[1]
        else:
            m = int(rng.integers(2, 65))
            k = int(rng.choice([1024, 4096, 4352, 12288]))
            rows = ("cus", int(rng.choice([1, 2, 3, 8])), int(rng.choice([-16, 0, 16])))
            n_est = 16 * 256 * rows[1]
        if m * n_est * k > 1.6e9:
            continue
        out.append((m, rows, k))
    return out


@pytest.mark.parametrize("m,rows,k", _random_batched_cases())
def test_batched_random_shapes(q4k, m, rows, k):
    """Every output written and inside the oracle's bound; where the header
    promises it (at least 16 rows per compute unit), two calls agree bitwise."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = rows[1] if rows[0] == "free" else max(1, 16 * cus * rows[1] + rows[2])
    print(f"[case] random batched m={m} {n}x{k}", flush=True)
    w = inputs.make_q4k(n, k, config_id=95, tensor_id=n + k)
    xs = inputs.make_x(m, k, config_id=95, tensor_id=m)
    wd, xd = to_dev(w.reshape(-1)), to_dev(xs)
    yd = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.gemv_batched(wd, xd, y=yd)
    y = to_host(yd)
    assert np.isfinite(y).all(), f"{int((~np.isfinite(y)).sum())} outputs not written"
    if n >= 16 * cus:
        assert torch.equal(yd, q4k.gemv_batched(wd, xd)), "two calls differ"
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    check_bound(y, yr, ar, f"random batched m={m} {n}x{k}")


@pytest.mark.parametrize("m,n,k", [(4, 70, 12288), (16, 70, 12288), (64, 70, 12288), (3, 10, 256), (20, 10, 256),
                                   (7, 129, 20480), (40, 129, 1280), (2, 70, 12288), (2, 129, 8192), (2, 33, 16384),
                                   (2, 300, 4352), (4, 4097, 1024), (3, 1, 256), (2, 5, 20480)])
def test_batched_shapes(q4k, m, n, k):
    w = inputs.make_q4k(n, k, config_id=97, tensor_id=k)
    xs = inputs.make_x(m, k, config_id=97, tensor_id=m)
    y = to_host(q4k.gemv_batched(to_dev(w.reshape(-1)), to_dev(xs)))
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    _report(f"batched m={m} {n}x{k}", check_bound(y, yr, ar, f"batched m={m} {n}x{k}"))


@pytest.mark.parametrize("name,tid", [("gate_9b", 0), ("down_9b", 2)])
@pytest.mark.parametrize("m", [1, 2, 4, 16, 32, 64])
def test_batched_ffn_9b_whole(q4k, name, tid, m):
    """Whole matrix on the GPU (y pre-filled with NaN: every output must be
    written), every output against the oracle."""
    import torch

    n, k = inputs.SHAPES[name]
    w = inputs.make_q4k(n, k, config_id=4, tensor_id=tid)
    xs = inputs.make_x(m, k, config_id=4, tensor_id=100 + m)
    yd = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.gemv_batched(to_dev(w.reshape(-1)), to_dev(xs), y=yd)
    y = to_host(yd)
    assert np.isfinite(y).all(), f"{int((~np.isfinite(y)).sum())} outputs not written"
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    _report(f"batched 9b {name} m={m}", check_bound(y, yr, ar, f"batched {name} m={m}"))


@pytest.mark.parametrize("m,n,k", [(2, 4096, 4096), (3, 1000, 4096), (4, 4097, 1024), (2, 777, 2048), (4, 300, 256),
                                   (2, 4096, 12288), (2, 1000, 8192), (2, 515, 16384)])
def test_batched_few_tokens_equal_batch1_bitwise(q4k, m, n, k):
    """Up to four tokens (two at K > 4096) run on the streaming GEMV kernels,
    which decode each weight group once for a pair of tokens and otherwise do
    per token exactly the arithmetic of the batch-1 call: every token's row
    equals q4k_gemv on that token bit for bit, and is inside the oracle's
    bound."""
    import torch

    print(f"[case] few tokens m={m} {n}x{k}", flush=True)
    assert batched_on_gemv_kernels(m, n, k)
    w = inputs.make_q4k(n, k, config_id=95, tensor_id=k)
    xs = inputs.make_x(m, k, config_id=95, tensor_id=m)
    wd, xd = to_dev(w.reshape(-1)), to_dev(xs)
    yd = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.gemv_batched(wd, xd, y=yd)
    for t in range(m):
        assert torch.equal(yd[t], q4k.gemv(wd, xd[t])), f"token {t} differs from the batch-1 call"
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    _report(f"few tokens m={m} {n}x{k}", check_bound(to_host(yd), yr, ar, f"few tokens m={m} {n}x{k}"))


@pytest.mark.parametrize("m,n,k", [(5, 4096, 256), (16, 4100, 1024), (9, 4096, 2048), (16, 4111, 2304),
                                   (12, 5000, 3328), (7, 4097, 4096), (16, 8192, 4096), (4, 16400, 1024),
                                   (3, 16384, 2048)])
def test_batched_streamed_tiles(q4k, m, n, k):
    """5 to 16 tokens with k <= 4096 and a 16-row tile for every CU, or 3 and
    4 tokens with four tiles per CU: the matrix-core kernel that streams the
    weights (each wave holding its K slice's activation operands), including
    waves whose last halves are past the row (k = 2304, 3328) and a ragged
    last tile.  Every output is written, inside the bound, and the same bits
    on a second run."""
    assert not batched_on_gemv_kernels(m, n, k)
    import torch

    print(f"[case] streamed tiles m={m} {n}x{k}", flush=True)
    w = inputs.make_q4k(n, k, config_id=94, tensor_id=k)
    xs = inputs.make_x(m, k, config_id=94, tensor_id=m)
    wd, xd = to_dev(w.reshape(-1)), to_dev(xs)
    yd = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.gemv_batched(wd, xd, y=yd)
    y = to_host(yd)
    assert np.isfinite(y).all(), f"{int((~np.isfinite(y)).sum())} outputs not written"
    assert torch.equal(q4k.gemv_batched(wd, xd), yd), "not reproducible"
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    _report(f"streamed m={m} {n}x{k}", check_bound(y, yr, ar, f"streamed m={m} {n}x{k}"))


def _boundary_cases():
    # the batched call's kernel choice switches at m = 2 | 3..4 | 5..16 | 17+,
    # at K = 4096 (token pairs, streamed tiles) and 16384 (two-token K split),
    # and at 16 and 64 rows per CU (rows as multiples of 16 * CUs, here for up
    # to 256 CUs: each side of each switch appears for any CU count <= 256);
    # rows longer than 4096 weights halve K between two workgroups at exactly
    # one 16-row tile per CU with no more than 32 rows per CU pair (4096 rows
    # on 256 CUs: 4080, 4096 and 4112 rows are its two sides)
    out = []
    for m in (2, 3, 4, 5, 16, 17):
        for n in (4080, 4096, 16368, 16384):
            out.append((m, n, 4096))
        out.append((m, 16384, 4352))
    for m in (3, 16, 17, 64):
        for n in (4080, 4096, 4112):
            out.append((m, n, 4352))
    # the streaming matrix-core kernel splits K = 4096 between two workgroups
    # up to 8 tiles per CU (32768 rows on 256 CUs)
    out += [(5, 32768, 4096), (16, 32784, 4096)]
    out += [(2, 512, 16384), (2, 512, 16640), (3, 512, 16384)]
    return out


@pytest.mark.parametrize("m,n,k", _boundary_cases())
def test_batched_kernel_choice_boundaries(q4k, m, n, k):
    """Both sides of every switch in the batched call's kernel choice: every
    output written, every output inside the oracle's bound, and the few-token
    path's rows equal to q4k_gemv per token."""
    import torch

    print(f"[case] boundary m={m} {n}x{k} gemv-kernels={batched_on_gemv_kernels(m, n, k)}", flush=True)
    w = inputs.make_q4k(n, k, config_id=93, tensor_id=n + k)
    xs = inputs.make_x(m, k, config_id=93, tensor_id=m)
    wd, xd = to_dev(w.reshape(-1)), to_dev(xs)
    yd = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
    q4k.gemv_batched(wd, xd, y=yd)
    y = to_host(yd)
    assert np.isfinite(y).all(), f"{int((~np.isfinite(y)).sum())} outputs not written"
    if batched_on_gemv_kernels(m, n, k):
        for t in range(m):
            assert torch.equal(yd[t], q4k.gemv(wd, xd[t])), f"token {t} differs from the batch-1 call"
    yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
    check_bound(y, yr, ar, f"boundary m={m} {n}x{k}")


@pytest.mark.parametrize("n", [64, 4096])
def test_batched_special_values(q4k, n):
    """m = 4: the streaming GEMV kernels (two token pairs); m = 16: the staged
    matrix-core kernel at n = 64, the weight-streaming one at n = 4096."""
    k = 1024
    w = inputs.make_q4k(n, k, config_id=98, tensor_id=0)
    for m in (4, 16):
        xs = inputs.make_x(m, k, config_id=98, tensor_id=m)
        xs[1] = 0.0
        xs[2] *= np.float32(1e-30)
        xs[3] = (xs[3] * np.exp2(np.random.default_rng(m).integers(-8, 9, k))).astype(np.float32)
        y = to_host(q4k.gemv_batched(to_dev(w.reshape(-1)), to_dev(xs)))
        assert np.all(y[1] == 0)
        yr, ar = oracle.gemv_batched(w, xs, threads=THREADS)
        _report(f"batched special m={m}", check_bound(y, yr, ar, f"batched special m={m}"))
        xs[0, 5] = np.inf
        y = to_host(q4k.gemv_batched(to_dev(w.reshape(-1)), to_dev(xs)))
        assert np.all(np.isnan(y[0])) and np.all(np.isfinite(y[1:]))


@pytest.mark.parametrize("m,tiles_per_cu,k", [(4, 1, 12288), (16, 1, 12288), (40, 1, 12288), (64, 1, 12288),
                                               (5, 3, 4096), (16, 3, 4096)])
def test_batched_two_k_halves_bitwise(q4k, m, tiles_per_cu, k):
    """K halved between two workgroups, the two partial tiles added into a
    zeroed y with f32 atomics: one 16-row tile per compute unit with rows longer
    than 4096 weights (the 9B down's 4096 x 12288 on 256 CUs: 32-row workgroups),
    and the weight-streaming kernel with few tiles per compute unit at K = 4096
    (the 9B gate, 3 tiles per CU).  Two addends give the same sum in either
    order, so repeated calls agree bitwise, also with an f16 output (summed in
    f32, then rounded); every output inside the oracle's bound."""
    import torch

    print(f"[case] two K halves m={m} tiles/CU={tiles_per_cu} k={k}", flush=True)
    n = 16 * tiles_per_cu * torch.cuda.get_device_properties(0).multi_processor_count
    wh = inputs.make_q4k(n, k, config_id=94, tensor_id=m)
    xh = inputs.make_x(m, k, config_id=94, tensor_id=m)
    w, xs = to_dev(wh.reshape(-1)), to_dev(xh)
    a = to_host(q4k.gemv_batched(w, xs))
    b = to_host(q4k.gemv_batched(w, xs))
    np.testing.assert_array_equal(a, b)
    c = q4k.gemv_batched_dt(w, xs, out_dtype=torch.float16)
    d = q4k.gemv_batched_dt(w, xs, out_dtype=torch.float16)
    assert torch.equal(c, d)
    yr, ar = oracle.gemv_batched(wh, xh, threads=THREADS)
    check_bound(a, yr, ar, f"two K halves m={m} k={k}")
    # the f16 output is the f32 sum rounded once: its error adds half an f16 ulp
    ch = to_host(c).astype(np.float64)
    assert np.all(np.abs(ch - yr) <= 2e-4 * ar + np.abs(yr) * 2.0**-11 + 2.0**-24), "f16 output outside the bound"


def test_batched_run_to_run(q4k):
    """With at least 16 rows per compute unit every workgroup covers the whole
    K range and stores its tile: bitwise reproducible.  With fewer rows the K
    range is split across workgroups and the partial tiles are added with f32
    atomics, so the last bits may change between runs while every run stays
    inside the bound."""
    import torch

    k = 1024
    n_big = 16 * torch.cuda.get_device_properties(0).multi_processor_count
    for n in (n_big, 512):
        wh = inputs.make_q4k(n, k, config_id=99, tensor_id=n)
        w = to_dev(wh.reshape(-1))
        for m in (4, 32):
            xh = inputs.make_x(m, k, config_id=99, tensor_id=m)
            xs = to_dev(xh)
            a = to_host(q4k.gemv_batched(w, xs))
            b = to_host(q4k.gemv_batched(w, xs))
            if n == n_big:
                np.testing.assert_array_equal(a, b)
            yr, ar = oracle.gemv_batched(wh, xh, threads=THREADS)
            check_bound(a, yr, ar, f"run 1 m={m} n={n}")
            check_bound(b, yr, ar, f"run 2 m={m} n={n}")