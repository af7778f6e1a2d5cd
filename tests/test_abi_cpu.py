"""The C ABI without a GPU: the library loads, exports what include/q4k.h
declares, and rejects bad arguments on the host before anything is launched
(every case here returns before the first HIP runtime call)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4k.h")


@pytest.fixture(scope="module")
def L():
    from q4_dequant_gemv_amd import q4k

    return q4k.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"Q4K_API\s+[\w\s\*]+?\b(q4k_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(
        ["q4k_gemv", "q4k_gemv_dt", "q4k_gemv_residual", "q4k_gemv_multi", "q4k_q8_0_gemv", "q4k_gemv_batched",
         "q4k_gemv_batched_dt", "q4k_gemv_batched_noalloc", "q4k_prefill_gemm", "q4k_gemv_batched_workspace_size",
         "q4k_gemv_batched_ws",
         "q4k_prefill_workspace_size", "q4k_prefill_gemm_ws", "q4k_fused_swiglu", "q4k_dequant",
         "q4k_status_string", "q4k_abi_version"])


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    from q4_dequant_gemv_amd import q4k

    assert sorted(q4k.EXPORTS) == declared_functions()


def test_only_the_abi_is_exported():
    import subprocess

    from q4_dequant_gemv_amd import q4k

    out = subprocess.run(["nm", "-D", "--defined-only", q4k.LIB_PATH], capture_output=True, text=True, check=True)
    names = {ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()}
    # HIP keeps kernel handles (C++ names in namespace q4k) and per-file ids
    # visible for its runtime registration; every C symbol is an ABI entry point
    c_names = {n for n in names if not n.startswith(("__hip_cuid", "_ZN3q4k"))}
    assert c_names == set(declared_functions())


def test_status_strings(L):
    assert L.q4k_abi_version() == 109
    assert re.search(r"#define Q4K_ABI_VERSION (\d+)", open(HEADER).read()).group(1) == "109"
    for s in range(5):
        assert len(L.q4k_status_string(s)) > 0
    assert L.q4k_status_string(99) == b"unknown status"


# fake, never dereferenced device addresses: validation must reject before use
A = 0x7F0000000000
W, X, Y, Y2 = A, A + 0x10000000, A + 0x20000000, A + 0x30000000
OK, INVALID, SHAPE, MISALIGNED = 0, 1, 2, 3


@pytest.mark.parametrize("args,status", [
    ((W, X, Y, 16, 300), SHAPE),                  # k % 256 != 0
    ((W, X, Y, -1, 256), INVALID),                # negative n
    ((W, X, Y, 16, -256), INVALID),               # negative k
    ((0, X, Y, 16, 256), INVALID),                # null w
    ((W, 0, Y, 16, 256), INVALID),                # null x
    ((W, X, 0, 16, 256), INVALID),                # null y
    ((W + 8, X, Y, 16, 256), MISALIGNED),         # w not 16-B aligned
    ((W, X + 2, Y, 16, 256), MISALIGNED),         # x not 4-B aligned
    ((W, X, Y + 1, 16, 256), MISALIGNED),         # y not 4-B aligned
    ((W, X, W + 64, 16, 256), INVALID),           # y overlaps w
    ((W, X, X, 16, 256), INVALID),                # y aliases x
    ((W, X, Y, 1 << 50, 1 << 20), INVALID),       # element count overflow
    ((W, X, Y, 0, 256), OK),                      # empty: nothing launched
    ((0, 0, 0, 0, 256), OK),
])
def test_gemv_validation(L, args, status):
    w, x, y, n, k = args
    assert L.q4k_gemv(ctypes.c_void_p(w), ctypes.c_void_p(x), ctypes.c_void_p(y), n, k, None) == status


R = A + 0x40000000


@pytest.mark.parametrize("args,status", [
    ((W, X, R, Y, 16, 300), SHAPE),
    ((W, X, 0, Y, 16, 256), INVALID),             # null residual
    ((W, X, R + 2, Y, 16, 256), MISALIGNED),
    ((W, X, Y + 4, Y, 16, 256), INVALID),         # r overlaps y without being y
    ((W, X, R, X + 4, 16, 256), INVALID),         # y overlaps x
    ((W, X, R, W, 16, 256), INVALID),             # y overlaps w
    ((W, X, R, Y, 0, 256), OK),
    ((0, 0, 0, 0, 0, 0), OK),
])
def test_residual_validation(L, args, status):
    w, x, r, y, n, k = args
    assert L.q4k_gemv_residual(ctypes.c_void_p(w), ctypes.c_void_p(x), ctypes.c_void_p(r), ctypes.c_void_p(y), n, k,
                               None) == status


@pytest.mark.parametrize("args,status", [
    ((W, X, Y, 16, 48), SHAPE),                   # k % 32 != 0
    ((W, X, Y, -1, 64), INVALID),
    ((W, X, Y, 16, -64), INVALID),
    ((0, X, Y, 16, 64), INVALID),
    ((W, 0, Y, 16, 64), INVALID),
    ((W, X, 0, 16, 64), INVALID),
    ((W + 1, X, Y, 16, 64), MISALIGNED),          # w must be 2-B aligned
    ((W, X + 2, Y, 16, 64), MISALIGNED),
    ((W, X, Y + 2, 16, 64), MISALIGNED),
    ((W, X, W + 16 * 68 - 4, 16, 64), INVALID),   # y overlaps the last bytes of w
    ((W, X, X + 252, 16, 64), INVALID),           # y overlaps x
    ((W, X, Y, 1 << 50, 1 << 20), INVALID),
    ((W, X, Y, 0, 64), OK),
    ((0, 0, 0, 0, 32), OK),
])
def test_q8_0_validation(L, args, status):
    w, x, y, n, k = args
    assert L.q4k_q8_0_gemv(ctypes.c_void_p(w), ctypes.c_void_p(x), ctypes.c_void_p(y), n, k, None) == status


@pytest.mark.parametrize("args,status", [
    ((W, X, 1, Y, 1, 16, 300), SHAPE),
    ((W, X, 2, Y, 0, 16, 256), INVALID),          # unknown dtype
    ((W, X, 0, Y, -1, 16, 256), INVALID),
    ((W, X + 2, 0, Y, 0, 16, 256), MISALIGNED),   # f32 x at 2-B
    ((W, X + 1, 1, Y, 1, 16, 256), MISALIGNED),   # f16 x at 1-B
    ((W, X, 1, Y + 1, 1, 16, 256), MISALIGNED),
    ((W, X, 1, Y + 2, 0, 16, 256), MISALIGNED),   # f32 y at 2-B
    ((W, X, 1, X + 510, 1, 16, 256), INVALID),    # f16 y overlaps the last f16 of x
    ((W, X, 0, Y, 1, 0, 256), OK),
])
def test_gemv_dt_validation(L, args, status):
    w, x, xd, y, yd, n, k = args
    assert L.q4k_gemv_dt(ctypes.c_void_p(w), ctypes.c_void_p(x), xd, ctypes.c_void_p(y), yd, n, k, None) == status


@pytest.mark.parametrize("args,status", [
    ((W, X, 1, Y, 1, 4, 16, 300), SHAPE),
    ((W, X, 3, Y, 1, 4, 16, 256), INVALID),
    ((W, X + 2, 0, Y, 1, 4, 16, 256), MISALIGNED),
    ((W, X, 1, Y + 2, 0, 4, 16, 256), MISALIGNED),
    ((W, X, 1, X + 4 * 256 * 2 - 2, 1, 4, 16, 256), INVALID),  # y starts inside f16 x[4, 256]
    ((W, X, 1, Y, 1, 0, 16, 256), OK),
    ((W, X, 1, Y, 1, -1, 16, 256), INVALID),
])
def test_batched_dt_validation(L, args, status):
    w, x, xd, y, yd, m, n, k = args
    assert L.q4k_gemv_batched_dt(ctypes.c_void_p(w), ctypes.c_void_p(x), xd, ctypes.c_void_p(y), yd, m, n, k,
                                 None) == status


@pytest.mark.parametrize("args,status", [
    ((W, X, 1, Y, 1, 4, 16, 300), SHAPE),
    ((W, X, 3, Y, 1, 4, 16, 256), INVALID),
    ((W, X + 2, 0, Y, 1, 4, 16, 256), MISALIGNED),
    ((W, X, 1, Y + 2, 0, 4, 16, 256), MISALIGNED),
    ((W, X, 1, X + 4 * 256 * 2 - 2, 1, 4, 16, 256), INVALID),  # y starts inside f16 x[4, 256]
    ((W, X, 1, Y, 1, 0, 16, 256), OK),
    ((W, X, 1, Y, 1, -1, 16, 256), INVALID),
    # scratch beyond the per-GPU array (4096 f16 tokens at k = 4096: the
    # prefill GEMM's 32 MiB of activation operands alone)
    ((W, X, 1, Y, 0, 4096, 4096, 4096), SHAPE),
])
def test_batched_noalloc_validation(L, args, status):
    w, x, xd, y, yd, m, n, k = args
    assert L.q4k_gemv_batched_noalloc(ctypes.c_void_p(w), ctypes.c_void_p(x), xd, ctypes.c_void_p(y), yd, m, n, k,
                                      None) == status


@pytest.mark.parametrize("args,status", [
    ((W, X, Y, 0, 128, 16, 300), SHAPE),
    ((W, X, Y, 0, 128, 16, (1 << 24) + 256), SHAPE),  # beyond the kernel's 32-bit row-block offsets
    ((W, X, Y, 2, 128, 16, 256), INVALID),           # unknown output dtype
    ((W, X, Y, 0, -1, 16, 256), INVALID),
    ((W, X + 8, Y, 0, 128, 16, 256), MISALIGNED),    # x must be 16-B aligned
    ((W + 8, X, Y, 0, 128, 16, 256), MISALIGNED),
    ((W, X, Y + 2, 0, 128, 16, 256), MISALIGNED),    # f32 y at 2-B
    ((W, X, Y + 1, 1, 128, 16, 256), MISALIGNED),
    ((W, X, X + 128 * 512 - 2, 1, 128, 16, 256), INVALID),  # f16 y starts inside x [128, 256] f16
    ((W, 0, Y, 0, 128, 16, 256), INVALID),
    ((W, X, Y, 0, 0, 16, 256), OK),
    ((W, X, Y, 1, 128, 0, 256), OK),
])
def test_prefill_validation(L, args, status):
    w, x, y, yd, m, n, k = args
    assert L.q4k_prefill_gemm(ctypes.c_void_p(w), ctypes.c_void_p(x), ctypes.c_void_p(y), yd, m, n, k, None) == status


WS = A + 0x40000000  # a 256-byte aligned stand-in workspace address


@pytest.mark.parametrize("args,status", [
    ((W, X, 1, Y, 1, 4, 16, 300, WS, 1 << 20), SHAPE),
    ((W, X, 3, Y, 1, 4, 16, 256, WS, 1 << 20), INVALID),
    ((W, X + 2, 0, Y, 1, 4, 16, 256, WS, 1 << 20), MISALIGNED),
    ((W, X, 1, X + 4 * 256 * 2 - 2, 1, 4, 16, 256, WS, 1 << 20), INVALID),
    ((W, X, 1, Y, 1, 4, 16, 256, WS, -1), INVALID),        # negative workspace size
    ((W, X, 1, Y, 1, 4, 16, 256, WS + 128, 1 << 20), MISALIGNED),  # workspace not 256-B aligned
    ((W, X, 1, Y, 1, 0, 16, 256, WS, -1), INVALID),        # checked even for an empty call
    ((W, X, 1, Y, 1, 0, 16, 256, 0, 0), OK),
    ((W, X, 1, Y, 1, 4, 0, 256, 0, 0), OK),
])
def test_batched_ws_validation(L, args, status):
    w, x, xd, y, yd, m, n, k, ws, wsb = args
    assert L.q4k_gemv_batched_ws(ctypes.c_void_p(w), ctypes.c_void_p(x), xd, ctypes.c_void_p(y), yd, m, n, k,
                                 ctypes.c_void_p(ws), wsb, None) == status


@pytest.mark.parametrize("args,status", [
    ((W, X, Y, 0, 128, 16, 300, WS, 1 << 20), SHAPE),
    ((W, X, Y, 0, 128, 16, (1 << 24) + 256, WS, 1 << 20), SHAPE),
    ((W, X + 8, Y, 0, 128, 16, 256, WS, 1 << 20), MISALIGNED),
    ((W, X, Y, 2, 128, 16, 256, WS, 1 << 20), INVALID),
    ((W, X, Y, 0, 128, 16, 256, WS, -5), INVALID),
    ((W, X, Y, 0, 128, 16, 256, WS + 16, 1 << 20), MISALIGNED),
    ((W, X, Y, 0, 0, 16, 256, 0, 0), OK),
])
def test_prefill_ws_validation(L, args, status):
    w, x, y, yd, m, n, k, ws, wsb = args
    assert L.q4k_prefill_gemm_ws(ctypes.c_void_p(w), ctypes.c_void_p(x), ctypes.c_void_p(y), yd, m, n, k,
                                 ctypes.c_void_p(ws), wsb, None) == status


def test_workspace_size_queries(L):
    out = ctypes.c_int64(-1)
    # sizes that need no device: empty calls, one token, k == 0,
    # and up to 4 tokens with k <= 4096 (the streaming GEMV kernel)
    for m, n, k in ((0, 16, 256), (4, 0, 256), (1, 4096, 4096), (8, 16, 0), (2, 16, 256), (4, 48, 4096)):
        for xd in (0, 1):
            for yd in (0, 1):
                out.value = -1
                assert L.q4k_gemv_batched_workspace_size(xd, yd, m, n, k, ctypes.byref(out)) == OK
                assert out.value == 0
    for m, n, k in ((0, 16, 256), (128, 0, 256), (128, 16, 0)):
        out.value = -1
        assert L.q4k_prefill_workspace_size(1, m, n, k, ctypes.byref(out)) == OK
        assert out.value == 0
    assert L.q4k_gemv_batched_workspace_size(0, 0, 4, 16, 256, None) == INVALID
    assert L.q4k_gemv_batched_workspace_size(2, 0, 4, 16, 256, ctypes.byref(out)) == INVALID
    assert L.q4k_gemv_batched_workspace_size(0, 0, 4, 16, 300, ctypes.byref(out)) == SHAPE
    assert L.q4k_gemv_batched_workspace_size(0, 0, -1, 16, 256, ctypes.byref(out)) == INVALID
    assert L.q4k_prefill_workspace_size(0, 128, 16, 256, None) == INVALID
    assert L.q4k_prefill_workspace_size(3, 128, 16, 256, ctypes.byref(out)) == INVALID
    assert L.q4k_prefill_workspace_size(0, 128, 16, (1 << 24) + 256, ctypes.byref(out)) == SHAPE
    assert L.q4k_prefill_workspace_size(0, -2, 16, 256, ctypes.byref(out)) == INVALID


def _items(*triples):
    """(w, y, n) or (w, y, n, y_gate, head_dim) per item."""
    from q4_dequant_gemv_amd import q4k

    items = (q4k.GemvItem * max(len(triples), 1))()
    for i, t in enumerate(triples):
        items[i].w, items[i].y, items[i].n = t[:3]
        if len(t) == 5:
            items[i].y_gate, items[i].head_dim = t[3:]
    return items


@pytest.mark.parametrize("triples,count,x,k,status", [
    ([(W, Y, 16)], 1, X, 300, SHAPE),
    ([(W, Y, 16)] * 9, 9, X, 256, INVALID),                      # more than Q4K_MAX_MULTI
    ([(W, Y, 16)], -1, X, 256, INVALID),
    ([(W, Y, 16), (Y2, Y, 16)], 2, X, 256, INVALID),             # two outputs alias
    ([(W, Y, 16), (Y2, Y + 60, 16)], 2, X, 256, INVALID),        # outputs overlap
    ([(W, Y, 16), (Y2, Y2 + 64, 16)], 2, X, 256, INVALID),       # an output overlaps another matrix
    ([(W, X, 16)], 1, X, 256, INVALID),                          # output aliases x
    ([(W, Y, 16), (0, Y2, 16)], 2, X, 256, INVALID),             # null matrix
    ([(W, Y, 16), (Y2, 0, 16)], 2, X, 256, INVALID),             # null output
    ([(W, Y, 16), (Y2 + 8, R, 16)], 2, X, 256, MISALIGNED),
    ([(W, Y, 16)], 1, 0, 256, INVALID),                          # null x
    ([(W, Y, -16)], 1, X, 256, INVALID),
    ([(W, Y, 0), (0, 0, 0)], 2, X, 256, OK),                     # no rows: nothing launched
    ([], 0, 0, 256, OK),
])
def test_multi_validation(L, triples, count, x, k, status):
    assert L.q4k_gemv_multi(_items(*triples), count, ctypes.c_void_p(x), k, None) == status


Y3 = A + 0x50000000


@pytest.mark.parametrize("triples,k,status", [
    ([(W, Y, 4096, Y3, 0)], 1024, INVALID),                     # head_dim must be positive
    ([(W, Y, 4096, Y3, 96)], 1024, INVALID),                    # not a power of two
    ([(W, Y, 4000, Y3, 256)], 1024, INVALID),                   # n not a multiple of 2 * head_dim
    ([(W, Y, 4096, Y3, 256)], 8192, SHAPE),                     # one launch only up to k = 4096
    ([(W, Y, 4096, Y + 8000, 256)], 1024, INVALID),             # gate half overlaps the q half
    ([(W, Y, 4096, Y3, 256), (Y2, Y3 + 4096, 16)], 1024, INVALID),  # another output inside the gate half
    ([(W, Y, 4096, W + 64, 256)], 1024, INVALID),               # gate output overlaps the matrix
    ([(W, Y, 4096, Y3 + 2, 256)], 1024, MISALIGNED),
    ([(W, Y, 0, Y3, 96)], 1024, OK),                            # empty item: nothing checked beyond the shape
])
def test_multi_split_qg_validation(L, triples, k, status):
    assert L.q4k_gemv_multi(_items(*triples), len(triples), ctypes.c_void_p(X), k, None) == status


def test_multi_null_items(L):
    assert L.q4k_gemv_multi(None, 1, ctypes.c_void_p(X), 256, None) == INVALID
    assert L.q4k_gemv_multi(None, 0, ctypes.c_void_p(X), 256, None) == OK


@pytest.mark.parametrize("args,status", [
    ((W, X, Y, 4, 16, 300), SHAPE),
    ((W, X, Y, -4, 16, 256), INVALID),
    ((W, X, Y, 4, 16, 256 + 8), SHAPE),
    ((W, 0, Y, 4, 16, 256), INVALID),
    ((W, X + 1, Y, 4, 16, 256), MISALIGNED),
    ((W, X, X + 4 * 256, 4, 16, 256), INVALID),   # y starts inside x[4, 256]
    ((W, X, Y, 0, 16, 256), OK),
    ((W, X, Y, 4, 0, 256), OK),
    ((W, X, Y, 1 << 40, 1 << 20, 1 << 20), INVALID),
])
def test_batched_validation(L, args, status):
    w, x, y, m, n, k = args
    assert L.q4k_gemv_batched(ctypes.c_void_p(w), ctypes.c_void_p(x), ctypes.c_void_p(y), m, n, k, None) == status


@pytest.mark.parametrize("args,status", [
    ((W, Y2, X, Y, 16, 300), SHAPE),
    ((W, 0, X, Y, 16, 256), INVALID),
    ((W, Y2 + 4, X, Y, 16, 256), MISALIGNED),
    ((W, Y2, X, Y2 + 16, 16, 256), INVALID),      # h overlaps w_up
    ((W, Y2, X, Y, 0, 256), OK),
])
def test_swiglu_validation(L, args, status):
    wg, wu, x, h, n, k = args
    assert L.q4k_fused_swiglu(ctypes.c_void_p(wg), ctypes.c_void_p(wu), ctypes.c_void_p(x), ctypes.c_void_p(h), n, k,
                              None) == status


@pytest.mark.parametrize("args,status", [
    ((W, Y, 16, 300), SHAPE),
    ((W, 0, 16, 256), INVALID),
    ((W, Y + 4, 16, 256), MISALIGNED),             # dequant output needs 16-B alignment
    ((W, W, 16, 256), INVALID),
    ((W, Y, 0, 256), OK),
    ((W, Y, 16, 0), OK),
])
def test_dequant_validation(L, args, status):
    w, out, n, k = args
    assert L.q4k_dequant(ctypes.c_void_p(w), ctypes.c_void_p(out), n, k, None) == status


def test_binding_never_falls_back(monkeypatch, tmp_path):
    """With the library missing the binding raises; it has no other path."""
    from q4_dequant_gemv_amd import q4k

    monkeypatch.setattr(q4k, "_lib", None)
    monkeypatch.setattr(q4k, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        q4k.lib()


def test_product_does_not_touch_the_oracle():
    """No file of the product package names the oracle."""
    pkg = os.path.join(ROOT, "q4_dequant_gemv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "q4k_oracle" not in text, f


def test_stream_read_probe_library():
    """The benchmark's read-only streaming kernel lives in a library of its
    own: it exports exactly its one C function and rejects bad arguments on
    the host (no device call is made for these)."""
    import subprocess

    from q4_dequant_gemv_amd import build as hip_build

    out = subprocess.run(["nm", "-D", "--defined-only", hip_build.STREAM_LIB], capture_output=True, text=True,
                         check=True)
    names = {ln.split()[-1] for ln in out.stdout.splitlines() if ln.strip()}
    assert {n for n in names if not n.startswith(("__hip_cuid", "_Z"))} == {"q4k_stream_read"}
    L = ctypes.CDLL(hip_build.STREAM_LIB)
    L.q4k_stream_read.restype = ctypes.c_int
    L.q4k_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    for args in ((0, 1024, Y, 8, 4, 0), (X, 1000, Y, 8, 4, 0), (X, 1 << 31, Y, 8, 4, 2), (X, 1024, 0, 8, 4, 0),
                 (X, 1024, Y, 0, 4, 2), (X, 1024, Y, 8, 5, 0), (X, -16, Y, 8, 8, 0), (X, 1024, Y, 8, 4, 1),
                 (X, 1024, Y, 8, 8, 3)):
        assert L.q4k_stream_read(*args, None) != 0, args
