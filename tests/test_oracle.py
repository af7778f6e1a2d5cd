"""Pins for the CPU oracle (runs without a GPU).

The oracle is checked against things other than itself:
  * a super-block worked by hand (tests/golden/q4k_single_block.txt) and two
    Q8_0 blocks worked by hand (tests/golden/q8_0_two_blocks.txt),
  * an independent bit-position decoder (tests/independent_decoder.py), and
    numpy's binary16 / int8 views for Q8_0,
  * IEEE binary16 decoding by numpy for all 65,536 patterns,
  * the inverse of the six-bit scale packing, exhaustively,
  * closed forms and invariants: zero codes give -dmin*m, linearity in x,
    integer matrices against an int64 numpy matmul (also with a residual
    added), exactness of the f32 dequant at the configs' value ranges, silu
    against scipy's expit.
``test_pins_catch_planted_mistakes`` plants plausible bugs in a copy of the
oracle source and checks that these pins reject every one.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import pytest
import scipy.special

import oracle as oracle_pkg
from golden_io import q8_0_two_blocks, single_block
from independent_decoder import codes as ind_codes
from independent_decoder import dequant as ind_dequant
from independent_decoder import pack_scales
from independent_decoder import scales_mins as ind_scales_mins
from q4_dequant_gemv_amd import inputs


# ---------------------------------------------------------------- helpers
def _blocks_f16(d, dmin, scales, qs):
    return inputs.assemble_blocks(np.asarray(qs, np.uint8), np.asarray(scales, np.uint8),
                                  np.asarray(d, np.float16), np.asarray(dmin, np.float16))


def _random_blocks(nb, seed, full_range_d=False):
    g = np.random.default_rng(seed)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    sc = g.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    if full_range_d:
        # finite f16 bit patterns of both signs, including subnormals
        bits = g.integers(0, 0x7C00, size=(nb, 2), dtype=np.uint16)
        bits |= (g.integers(0, 2, size=(nb, 2), dtype=np.uint16) << 15)
        d = bits[:, 0].view(np.float16)
        dmin = bits[:, 1].view(np.float16)
    else:
        d = g.uniform(1e-3, 1e-2, nb).astype(np.float16)
        dmin = g.uniform(1e-3, 1e-2, nb).astype(np.float16)
    return _blocks_f16(d, dmin, sc, qs)


# ------------------------------------------------------------- the pins
def check_golden_block(orc):
    gb = single_block()
    blk = gb["block"]
    for j, (sc, m) in enumerate(gb["scale_min"]):
        assert orc.scale_min(blk[4:16], j) == (sc, m), f"scale/min of sub-block {j}"
    w = orc.dequant_block(blk)
    for k, v in gb["weights"].items():
        assert w[k] == np.float32(v), f"w[{k}] = {w[k]}, hand value {v}"
    sums = w.astype(np.float64).reshape(8, 32).sum(axis=1)
    np.testing.assert_array_equal(sums, gb["subblock_sums"])
    wk = np.frombuffer(blk, np.uint8)
    y, a = orc.gemv(wk, np.ones(256, np.float32))
    assert y[0] == gb["y_ones"] and a[0] == gb["a_ones"]
    alt = np.where(np.arange(256) % 2 == 0, 1.0, -1.0).astype(np.float32)
    y, _ = orc.gemv(wk, alt)
    assert y[0] == gb["y_alternating"]
    y, _ = orc.gemv(wk, np.arange(256, dtype=np.float32))
    assert y[0] == gb["y_index"]


def check_independent_decoder(orc):
    for seed, full in ((1, False), (2, True)):
        blocks = _random_blocks(4000, seed, full_range_d=full)
        got = orc.dequant(blocks.reshape(-1), 256)
        want = ind_dequant(blocks)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    # dense f64 matvec on rows of 8 blocks (K=2048)
    blocks = _random_blocks(64 * 8, 3)
    x = np.random.default_rng(4).standard_normal(2048).astype(np.float32)
    y, a = orc.gemv(blocks.reshape(-1), x)
    wd = ind_dequant(blocks).reshape(64, 2048).astype(np.float64)
    yd = wd @ x.astype(np.float64)
    ad = np.abs(wd * x.astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(y, yd, rtol=0, atol=1e-12 * ad.max())
    np.testing.assert_allclose(a, ad, rtol=1e-13)


def check_zero_codes(orc):
    # all-zero nibbles: every weight is exactly -dmin*m of its sub-block
    blocks = _random_blocks(512, 5)
    blocks[:, 16:] = 0
    w = orc.dequant(blocks.reshape(-1), 256)
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float32)[:, 0]
    _, m = ind_scales_mins(blocks)
    ml = dmin[:, None] * m.astype(np.float32)
    np.testing.assert_array_equal(w, -np.repeat(ml, 32, axis=1))
    # y = -sum_s ml_s * sum_{k in s} x_k, exact with small-integer x
    x = np.random.default_rng(6).integers(-3, 4, 256).astype(np.float32)
    y, _ = orc.gemv(blocks.reshape(-1), x)
    want = -(ml.astype(np.float64) * x.reshape(8, 32).sum(axis=1)).sum(axis=1)
    np.testing.assert_array_equal(y, want)


def check_linearity(orc):
    blocks = _random_blocks(32 * 4, 7)
    g = np.random.default_rng(8)
    x1 = g.integers(-8, 9, 1024).astype(np.float32)
    x2 = g.integers(-8, 9, 1024).astype(np.float32)
    y1, _ = orc.gemv(blocks.reshape(-1), x1)
    y2, _ = orc.gemv(blocks.reshape(-1), x2)
    y3, _ = orc.gemv(blocks.reshape(-1), (2 * x1 - 4 * x2).astype(np.float32))
    np.testing.assert_array_equal(y3, 2 * y1 - 4 * y2)


def _integer_blocks(nb, seed):
    # d = 1, dmin = 0, every scale 1: the weight is the code itself
    g = np.random.default_rng(seed)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    sc = np.frombuffer(pack_scales([1] * 8, [g.integers(0, 64) for _ in range(8)]), np.uint8)
    return _blocks_f16(np.ones(nb), np.zeros(nb), np.tile(sc, (nb, 1)), qs)


def check_integer_matrix(orc):
    n, k, m = 48, 1024, 3
    blocks = _integer_blocks(n * k // 256, 9)
    q = ind_codes(blocks).reshape(n, k)
    g = np.random.default_rng(10)
    xs = g.integers(-50, 51, size=(m, k))
    y, _ = orc.gemv(blocks.reshape(-1), xs[0].astype(np.float32))
    np.testing.assert_array_equal(y, (q @ xs[0]).astype(np.float64))
    yb, _ = orc.gemv_batched(blocks.reshape(-1), xs.astype(np.float32))
    np.testing.assert_array_equal(yb, (xs @ q.T).astype(np.float64))
    # silu * up on exact integer g, u against scipy's logistic function
    blocks_u = _integer_blocks(n * k // 256, 11)
    qu = ind_codes(blocks_u).reshape(n, k)
    xsw = (xs[1] / 64.0).astype(np.float32)  # keeps g in a range where silu bends
    out = orc.fused_swiglu(blocks.reshape(-1), blocks_u.reshape(-1), xsw)
    gref = q @ xsw.astype(np.float64)
    uref = qu @ xsw.astype(np.float64)
    np.testing.assert_array_equal(out["g"], gref)
    np.testing.assert_array_equal(out["u"], uref)
    np.testing.assert_allclose(out["h"], gref * scipy.special.expit(gref) * uref, rtol=1e-14, atol=0)


def check_closed_form(orc):
    # at the configs' value ranges every f32 dequant step is exact
    blocks = _random_blocks(3000, 12)
    w = orc.dequant(blocks.reshape(-1), 256).astype(np.float64)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float64)[:, 0]
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float64)[:, 0]
    sc, m = ind_scales_mins(blocks)
    q = ind_codes(blocks)
    sub = np.arange(256) // 32
    exact = d[:, None] * sc[:, sub] * q - dmin[:, None] * m[:, sub]
    np.testing.assert_array_equal(w, exact)


def check_one_hot(orc):
    # code v at position e, zeros elsewhere, for all v and e
    nb = 16 * 256
    v = np.repeat(np.arange(16), 256)
    e = np.tile(np.arange(256), 16)
    qs = np.zeros((nb, 128), np.uint8)
    byte = 32 * (e // 64) + (e % 32)
    qs[np.arange(nb), byte] = np.where((e % 64) >= 32, v << 4, v).astype(np.uint8)
    scales = np.frombuffer(pack_scales([3, 5, 7, 11, 13, 17, 19, 23], [2, 4, 6, 8, 10, 12, 14, 16]), np.uint8)
    blocks = _blocks_f16(np.full(nb, 0.5), np.full(nb, 0.25), np.tile(scales, (nb, 1)), qs)
    w = orc.dequant(blocks.reshape(-1), 256)
    sc = np.array([3, 5, 7, 11, 13, 17, 19, 23], np.float64)
    mm = np.array([2, 4, 6, 8, 10, 12, 14, 16], np.float64)
    base = -0.25 * np.repeat(mm, 32)
    want = np.tile(base, (nb, 1))
    want[np.arange(nb), e] = 0.5 * sc[e // 32] * v - 0.25 * mm[e // 32]
    np.testing.assert_array_equal(w.astype(np.float64), want)


def check_residual(orc):
    # integer weights and activations with a residual of halves: every sum is
    # exact in f64, so y must equal the int64 product plus r exactly
    n, k = 40, 512
    blocks = _integer_blocks(n * k // 256, 16)
    q = ind_codes(blocks).reshape(n, k)
    g = np.random.default_rng(17)
    x = g.integers(-20, 21, k)
    r = (g.integers(-4000, 4001, n) / 2.0).astype(np.float32)
    y, a = orc.gemv_residual(blocks.reshape(-1), x.astype(np.float32), r)
    np.testing.assert_array_equal(y, (q @ x).astype(np.float64) + r.astype(np.float64))
    np.testing.assert_array_equal(a, (np.abs(q * x[None, :])).sum(axis=1).astype(np.float64)
                                  + np.abs(r.astype(np.float64)))
    # x = 0: the product vanishes and the residual passes through unchanged
    y0, _ = orc.gemv_residual(blocks.reshape(-1), np.zeros(k, np.float32), r)
    np.testing.assert_array_equal(y0, r.astype(np.float64))
    # the several-matrix form is one plain GEMV per matrix
    b2 = _integer_blocks(7 * k // 256, 18)
    q2 = ind_codes(b2).reshape(7, k)
    outs = orc.gemv_multi([blocks.reshape(-1), b2.reshape(-1)], x.astype(np.float32))
    np.testing.assert_array_equal(outs[0][0], (q @ x).astype(np.float64))
    np.testing.assert_array_equal(outs[1][0], (q2 @ x).astype(np.float64))


def check_row_ranges(orc):
    # rows [r0, r1) of a matrix with several super-blocks per row, r0 > 0:
    # the output starts at the first requested row, each block lands at its
    # own columns, and nothing is written past the requested rows (a guard
    # region after them keeps its sentinel)
    lib = orc._load()
    for k, seed in ((512, 40), (4096, 41)):
        n, r0, r1 = 11, 3, 9
        blocks = _random_blocks(n * k // 256, seed)
        rows = np.ascontiguousarray(blocks.reshape(n, -1))
        want = ind_dequant(blocks).reshape(n, k)
        buf = np.full((r1 + 1) * k, np.float32(-12345.5), dtype=np.float32)
        lib.q4k_oracle_dequant_rows(rows.ctypes.data, k, r0, r1, buf.ctypes.data)
        got = buf[:(r1 - r0) * k].reshape(r1 - r0, k)
        np.testing.assert_array_equal(got.view(np.uint32), want[r0:r1].view(np.uint32))
        assert np.all(buf[(r1 - r0) * k:] == np.float32(-12345.5)), "rows written past the requested range"
        # the threaded wrapper splits the rows into ranges with r0 > 0
        np.testing.assert_array_equal(orc.dequant(rows.reshape(-1), k, threads=3).view(np.uint32),
                                      want.view(np.uint32))


def check_batched_magnitudes(orc):
    # Y and the magnitude sums A of the batched call against a dense f64
    # product of independently decoded weights, token by token
    n, k, m = 24, 1024, 3
    blocks = _random_blocks(n * k // 256, 42)
    xs = np.random.default_rng(43).standard_normal((m, k)).astype(np.float32)
    y, a = orc.gemv_batched(blocks.reshape(-1), xs)
    wd = ind_dequant(blocks).reshape(n, k).astype(np.float64)
    xd = xs.astype(np.float64)
    want_a = np.abs(wd[None, :, :] * xd[:, None, :]).sum(axis=-1)
    assert a.shape == (m, n)
    np.testing.assert_allclose(a, want_a, rtol=1e-13, atol=0)
    np.testing.assert_allclose(y, xd @ wd.T, rtol=0, atol=1e-12 * want_a.max())


def check_swiglu_magnitudes(orc):
    # g, u and their magnitude sums ag, au against dense f64 products of two
    # different, independently decoded matrices (a swap of the two is caught)
    n, k = 20, 1024
    bg = _random_blocks(n * k // 256, 44)
    bu = _random_blocks(n * k // 256, 45)
    x = np.random.default_rng(46).standard_normal(k).astype(np.float32)
    out = orc.fused_swiglu(bg.reshape(-1), bu.reshape(-1), x)
    xd = x.astype(np.float64)
    for mat, val, mag in ((bg, "g", "ag"), (bu, "u", "au")):
        wd = ind_dequant(mat).reshape(n, k).astype(np.float64)
        want_a = np.abs(wd * xd[None, :]).sum(axis=1)
        np.testing.assert_allclose(out[mag], want_a, rtol=1e-13, atol=0)
        np.testing.assert_allclose(out[val], wd @ xd, rtol=0, atol=1e-12 * want_a.max())


# ------------------------------------------------------------------- Q8_0
def _q8_numpy_dequant(blocks):
    # independent of the oracle: numpy's binary16 and int8 views of the bytes
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float32)
    q = blocks[:, 2:].copy().view(np.int8).astype(np.float32)
    return d * q


def check_q8_golden(orc):
    gb = q8_0_two_blocks()
    row = np.frombuffer(gb["row"], np.uint8)
    w = orc.q8_0_dequant(row, 64)[0]
    for k, v in gb["weights"].items():
        assert w[k] == np.float32(v), f"q8 w[{k}] = {w[k]}, hand value {v}"
    y, a = orc.q8_0_gemv(row, np.ones(64, np.float32))
    assert y[0] == gb["y_ones"] and a[0] == gb["a_ones"]
    alt = np.where(np.arange(64) % 2 == 0, 1.0, -1.0).astype(np.float32)
    assert orc.q8_0_gemv(row, alt)[0][0] == gb["y_alternating"]
    assert orc.q8_0_gemv(row, np.arange(64, dtype=np.float32))[0][0] == gb["y_index"]


def check_q8_independent_decoder(orc):
    g = np.random.default_rng(31)
    nb = 20000
    q = g.integers(-128, 128, size=(nb, 32), dtype=np.int8)  # -128 included
    bits = g.integers(0, 0x7C00, size=nb, dtype=np.uint16) | (g.integers(0, 2, size=nb, dtype=np.uint16) << 15)
    blocks = inputs.assemble_q8_0(q, bits.view(np.float16))
    got = orc.q8_0_dequant(blocks.reshape(-1), 32)
    np.testing.assert_array_equal(got.view(np.uint32), _q8_numpy_dequant(blocks).view(np.uint32))
    # dense f64 matvec over rows of 32 blocks (K = 1024)
    w = inputs.make_q8_0(48, 1024, config_id=0, tensor_id=32)
    x = g.standard_normal(1024).astype(np.float32)
    wd = _q8_numpy_dequant(w.reshape(-1, 34)).reshape(48, 1024).astype(np.float64)
    y, a = orc.q8_0_gemv(w, x)
    np.testing.assert_allclose(y, wd @ x.astype(np.float64), rtol=0, atol=1e-12 * np.abs(wd * x).sum(axis=1).max())
    np.testing.assert_allclose(a, np.abs(wd * x.astype(np.float64)).sum(axis=1), rtol=1e-13)


def check_q8_integer_matrix(orc):
    # d = 1: the weights are the codes; y equals an int64 matmul exactly
    n, k = 40, 1024
    g = np.random.default_rng(33)
    q = g.integers(-128, 128, size=(n * k // 32, 32), dtype=np.int8)
    w = inputs.assemble_q8_0(q, np.ones(n * k // 32, np.float16)).reshape(n, -1)
    x = g.integers(-60, 61, k)
    y, a = orc.q8_0_gemv(w, x.astype(np.float32))
    qi = q.astype(np.int64).reshape(n, k)
    np.testing.assert_array_equal(y, (qi @ x).astype(np.float64))
    np.testing.assert_array_equal(a, np.abs(qi * x[None, :]).sum(axis=1).astype(np.float64))


ALL_PINS = [check_golden_block, check_independent_decoder, check_zero_codes, check_linearity,
            check_integer_matrix, check_closed_form, check_one_hot, check_residual, check_row_ranges,
            check_batched_magnitudes, check_swiglu_magnitudes,
            check_q8_golden, check_q8_independent_decoder, check_q8_integer_matrix]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, pin):
    pin(oracle_mod)


def test_f16_exhaustive(oracle_mod):
    lib = oracle_mod._load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    got = np.array([lib.q4k_oracle_f16_to_f32(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_scale_packing_exhaustive(oracle_mod):
    g = np.random.default_rng(13)
    for j in range(8):
        for sc in range(64):
            for m in range(64):
                scs = list(g.integers(0, 64, 8))
                ms = list(g.integers(0, 64, 8))
                scs[j], ms[j] = sc, m
                packed = pack_scales(scs, ms)
                assert oracle_mod.scale_min(packed, j) == (sc, m)


def test_packing_is_bijection():
    # every 12-byte pattern decodes to 16 six-bit values that pack back to it
    g = np.random.default_rng(14)
    raw = g.integers(0, 256, size=(5000, 144), dtype=np.uint8)
    sc, m = ind_scales_mins(raw)
    for i in range(raw.shape[0]):
        assert pack_scales(list(sc[i]), list(m[i])) == raw[i, 4:16].tobytes()


def test_threads_do_not_change_results(oracle_mod):
    w = inputs.make_q4k(257, 1024, config_id=0, tensor_id=1)
    x = inputs.make_x(1, 1024, config_id=0)[0]
    y1, a1 = oracle_mod.gemv(w, x, threads=1)
    y4, a4 = oracle_mod.gemv(w, x, threads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(a1, a4)
    yb, _ = oracle_mod.gemv_batched(w, np.stack([x, -x]), threads=3)
    np.testing.assert_array_equal(yb[0], y1)
    np.testing.assert_array_equal(yb[1], -y1)


def test_split_qg_pins(oracle_mod):
    """The per-head de-interleave ("@simulatte/doppler 0.1.7 -> 0.1.8",
    kernels/split_qg.wgsl): q[h*D + d] = y[h*2D + d], gate[h*D + d] =
    y[h*2D + D + d]."""
    # worked by hand: two heads of D = 2 over y = 0..7
    q, g = oracle_mod.split_qg(np.arange(8.0), 2)
    np.testing.assert_array_equal(q, [0, 1, 4, 5])
    np.testing.assert_array_equal(g, [2, 3, 6, 7])
    # one head: q is the first half of the rows, the gate the second
    y = np.random.default_rng(0).standard_normal(512)
    q, g = oracle_mod.split_qg(y, 256)
    np.testing.assert_array_equal(q, y[:256])
    np.testing.assert_array_equal(g, y[256:])
    # the split is a bijection: interleaving q and gate head by head gives y back
    y = np.random.default_rng(1).standard_normal(8 * 2 * 64)
    q, g = oracle_mod.split_qg(y, 64)
    back = np.stack([q.reshape(8, 64), g.reshape(8, 64)], axis=1).reshape(-1)
    np.testing.assert_array_equal(back, y)
    with pytest.raises(ValueError):
        oracle_mod.split_qg(np.zeros(300), 64)


def test_silu_special_cases(oracle_mod):
    # one-row matrices whose g is fixed: silu(0) = 0, silu(t) ~ t, silu(-t) ~ 0
    blocks = _integer_blocks(1, 15)
    q = ind_codes(blocks).reshape(-1).astype(np.float64)
    for scale, expect in ((0.0, "zero"), (1e3, "pos"), (-1e3, "neg")):
        x = np.zeros(256, np.float32)
        if scale:
            x[:] = scale / q.sum()
            x = x.astype(np.float32)
        out = oracle_mod.fused_swiglu(blocks.reshape(-1), blocks.reshape(-1), x)
        g, u, h = out["g"][0], out["u"][0], out["h"][0]
        if expect == "zero":
            assert h == 0.0
        elif expect == "pos":
            assert abs(h - g * u) <= 1e-12 * abs(g * u)
        else:
            assert abs(h) < 1e-300


# ----------------------------------------------- planted mistakes must fail
MUTATIONS = {
    "min_sign_flipped": ("out[e] = t - ml;", "out[e] = t + ml;"),
    "min_dropped": ("out[e] = t - ml;", "out[e] = t;"),
    "nibble_halves_swapped": ("return r < 32 ? (byte & 15) : (byte >> 4);",
                              "return r < 32 ? (byte >> 4) : (byte & 15);"),
    "high_scale_bits_from_wrong_byte": ("((scales[j - 4] >> 6) << 4)", "((scales[j] >> 6) << 4)"),
    "min_of_low_subblocks_wrong_byte": ("*m = scales[j + 4] & 63;", "*m = scales[j] & 63;"),
    "d_dmin_swapped": ("const float d = q4k_oracle_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));",
                       "const float d = q4k_oracle_f16_to_f32((uint16_t)(blk[2] | (blk[3] << 8)));"),
    "f16_bias_off_by_one": ("exponent - 25", "exponent - 24"),
    "group_stride_wrong": ("qs[32 * g + (r % 32)]", "qs[16 * g + (r % 32)]"),
    "x_index_transposed": ("x[b * Q4K_BLOCK_WEIGHTS + e]", "x[e * nb + b]"),
    "abs_sum_signed": ("mag += fabs(p);", "mag += p;"),
    "min_uses_scale": ("const float ml = dmin * (float)m;", "const float ml = dmin * (float)sc;"),
    "subblock_of_weight_wrong": ("const int j = e / 32; /* sub-block */", "const int j = (e % 128) / 16; /* sub-block */"),
    "silu_sign": ("exp(-g[i])", "exp(g[i])"),
    "residual_dropped": ("y[r - r0] = dot + (double)res[r];", "y[r - r0] = dot;"),
    "residual_subtracted": ("y[r - r0] = dot + (double)res[r];", "y[r - r0] = dot - (double)res[r];"),
    "residual_row_shifted": ("y[r - r0] = dot + (double)res[r];", "y[r - r0] = dot + (double)res[r1 - 1 - r];"),
    "q8_codes_unsigned": ("const int q = (int)(int8_t)blk[2 + e];", "const int q = (int)blk[2 + e];"),
    "q8_scale_bytes_swapped": ("(uint16_t)((blk[1] << 8) | blk[0])", "(uint16_t)((blk[0] << 8) | blk[1])"),
    "q8_codes_off_by_one": ("(int8_t)blk[2 + e]", "(int8_t)blk[1 + e]"),
    "q8_block_stride": ("q8_0_oracle_dequant_block(w + r * row_bytes + b * Q8_0_BLOCK_BYTES, wblk);",
                        "q8_0_oracle_dequant_block(w + r * row_bytes + b * Q8_0_BLOCK_WEIGHTS, wblk);"),
    "q8_x_index": ("x[b * Q8_0_BLOCK_WEIGHTS + e]", "x[e * nb + b]"),
    "q8_abs_signed": ("mag += p < 0.0 ? -p : p;", "mag += p;"),
    "rows_block_offset_in_bytes": ("out + (r - r0) * k + b * Q4K_BLOCK_WEIGHTS);",
                                   "out + (r - r0) * k + b * Q4K_BLOCK_BYTES);"),
    "rows_output_not_relative": ("out + (r - r0) * k + b * Q4K_BLOCK_WEIGHTS);", "out + r * k + b * Q4K_BLOCK_WEIGHTS);"),
    "batched_magnitude_transposed": ("&a[t * nr + (r - r0)]", "&a[(r - r0) * m + t]"),
    "swiglu_magnitudes_swapped": ("&g[i], &ag[i]);\n        q4k_oracle_row_dot(wu + r * row_bytes, k, x, &u[i], &au[i]);",
                                  "&g[i], &au[i]);\n        q4k_oracle_row_dot(wu + r * row_bytes, k, x, &u[i], &ag[i]);"),
}


def _run_pins_with(lib):
    saved = oracle_pkg._lib
    oracle_pkg._lib = lib
    try:
        failures = 0
        for pin in ALL_PINS + [lambda o: test_silu_special_cases(o)]:
            try:
                pin(oracle_pkg)
            except AssertionError:
                failures += 1
        return failures
    finally:
        oracle_pkg._lib = saved


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistakes(oracle_mod, name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle_pkg.__file__), "q4k_oracle.c")).read()
    assert before in src, f"mutation anchor for {name} not found"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(before, after))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared",
                           str(mutated), "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    # reuse the argtypes of the real library
    real = oracle_mod._load()
    for fn in ("q4k_oracle_f16_to_f32", "q4k_oracle_scale_min", "q4k_oracle_dequant_block",
               "q4k_oracle_dequant_rows", "q4k_gemv_oracle_into", "q4k_gemv_batched_oracle_into",
               "q4k_fused_swiglu_oracle_into", "q4k_gemv_residual_oracle_into", "q8_0_oracle_dequant_block",
               "q8_0_oracle_dequant_rows", "q8_0_gemv_oracle_into"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    assert _run_pins_with(lib) > 0, f"no pin caught the planted mistake {name}"
    # and the real oracle passes them all
    assert _run_pins_with(real) == 0
