"""Q4_K CPU oracle -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``q4k_oracle.c`` (plain C, f32 dequant, f64 dot).
Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library
(``q4_dequant_gemv_amd``) never imports, links or calls it, and the two share
no code: only the seeded input generators in
``q4_dequant_gemv_amd/inputs.py`` feed both.

Row ranges are split over host threads (``threads``); each thread runs the
unmodified C row loop on its own rows, so results do not depend on the thread
count.

Parity pins for every function live in ``tests/test_oracle.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4k_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BLOCK_BYTES = 144
BLOCK_WEIGHTS = 256
Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
             "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.q4k_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.q4k_oracle_f16_to_f32.restype = ctypes.c_float
        lib.q4k_oracle_scale_min.argtypes = [p, ctypes.c_int, p, p]
        lib.q4k_oracle_scale_min.restype = None
        lib.q4k_oracle_dequant_block.argtypes = [p, p]
        lib.q4k_oracle_dequant_block.restype = None
        lib.q4k_oracle_dequant_rows.argtypes = [p, i64, i64, i64, p]
        lib.q4k_oracle_dequant_rows.restype = None
        lib.q4k_gemv_oracle_into.argtypes = [p, p, i64, i64, i64, p, p]
        lib.q4k_gemv_oracle_into.restype = None
        lib.q4k_gemv_batched_oracle_into.argtypes = [p, p, i64, i64, i64, i64, p, p]
        lib.q4k_gemv_batched_oracle_into.restype = None
        lib.q4k_fused_swiglu_oracle_into.argtypes = [p, p, p, i64, i64, i64, p, p, p, p, p]
        lib.q4k_fused_swiglu_oracle_into.restype = None
        lib.q4k_gemv_residual_oracle_into.argtypes = [p, p, p, i64, i64, i64, p, p]
        lib.q4k_gemv_residual_oracle_into.restype = None
        lib.q8_0_oracle_dequant_block.argtypes = [p, p]
        lib.q8_0_oracle_dequant_block.restype = None
        lib.q8_0_oracle_dequant_rows.argtypes = [p, i64, i64, i64, p]
        lib.q8_0_oracle_dequant_rows.restype = None
        lib.q8_0_gemv_oracle_into.argtypes = [p, p, i64, i64, i64, p, p]
        lib.q8_0_gemv_oracle_into.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_rows(w: np.ndarray, k: int) -> np.ndarray:
    if k % BLOCK_WEIGHTS != 0:
        raise ValueError(f"k={k} is not a multiple of {BLOCK_WEIGHTS}")
    row_bytes = (k // BLOCK_WEIGHTS) * BLOCK_BYTES
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    if row_bytes == 0 or w.size % row_bytes != 0:
        raise ValueError("weight byte count is not a whole number of rows")
    return w.reshape(-1, row_bytes)


def _split(n: int, threads: int):
    threads = max(1, min(threads, n))
    bounds = np.linspace(0, n, threads + 1).astype(np.int64)
    return [(int(bounds[i]), int(bounds[i + 1])) for i in range(threads) if bounds[i] < bounds[i + 1]]


def _run(fn, n: int, threads: int):
    parts = _split(n, threads)
    if len(parts) == 1:
        fn(*parts[0])
        return
    with ThreadPoolExecutor(max_workers=len(parts)) as ex:
        list(ex.map(lambda ab: fn(*ab), parts))


def f16_to_f32(h: int) -> float:
    return float(_load().q4k_oracle_f16_to_f32(int(h) & 0xFFFF))


def scale_min(scales12: bytes, j: int) -> tuple[int, int]:
    buf = np.frombuffer(bytes(scales12), dtype=np.uint8).copy()
    sc = ctypes.c_int()
    m = ctypes.c_int()
    _load().q4k_oracle_scale_min(_ptr(buf), j, ctypes.byref(sc), ctypes.byref(m))
    return sc.value, m.value


def dequant_block(block144: bytes) -> np.ndarray:
    buf = np.frombuffer(bytes(block144), dtype=np.uint8).copy()
    if buf.size != BLOCK_BYTES:
        raise ValueError("a Q4_K super-block is 144 bytes")
    out = np.empty(BLOCK_WEIGHTS, dtype=np.float32)
    _load().q4k_oracle_dequant_block(_ptr(buf), _ptr(out))
    return out


def dequant(w: np.ndarray, k: int, threads: int = 1) -> np.ndarray:
    """W as f32 [n, k]."""
    rows = _as_rows(w, k)
    n = rows.shape[0]
    out = np.empty((n, k), dtype=np.float32)
    lib = _load()
    _run(lambda a, b: lib.q4k_oracle_dequant_rows(_ptr(rows), k, a, b, _ptr(out[a:b])), n, threads)
    return out


def gemv(w: np.ndarray, x: np.ndarray, threads: int = 1):
    """(y, A): y[n] = sum_k W[n,k] x[k] (f64), A[n] = sum_k |W[n,k] x[k]|."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    k = x.size
    rows = _as_rows(w, k)
    n = rows.shape[0]
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    lib = _load()
    _run(lambda r0, r1: lib.q4k_gemv_oracle_into(_ptr(rows[r0:r1]), _ptr(x), k, 0, r1 - r0,
                                                 _ptr(y[r0:r1]), _ptr(a[r0:r1])), n, threads)
    return y, a


def gemv_batched(w: np.ndarray, xs: np.ndarray, threads: int = 1):
    """(Y, A) of shape [m, n]: Y[t, n] = sum_k W[n,k] X[t,k] (f64)."""
    xs = np.ascontiguousarray(xs, dtype=np.float32)
    if xs.ndim != 2:
        raise ValueError("X must be [m, k]")
    m, k = xs.shape
    rows = _as_rows(w, k)
    n = rows.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    a = np.empty((m, n), dtype=np.float64)
    lib = _load()

    def part(r0, r1):
        yp = np.empty((m, r1 - r0), dtype=np.float64)
        ap = np.empty((m, r1 - r0), dtype=np.float64)
        lib.q4k_gemv_batched_oracle_into(_ptr(rows[r0:r1]), _ptr(xs), m, k, 0, r1 - r0, _ptr(yp), _ptr(ap))
        y[:, r0:r1] = yp
        a[:, r0:r1] = ap

    _run(part, n, threads)
    return y, a


def fused_swiglu(wg: np.ndarray, wu: np.ndarray, x: np.ndarray, threads: int = 1):
    """dict with h, g, u, ag, au (all f64 [n])."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    k = x.size
    rg = _as_rows(wg, k)
    ru = _as_rows(wu, k)
    if rg.shape != ru.shape:
        raise ValueError("gate and up matrices must have the same shape")
    n = rg.shape[0]
    out = {name: np.empty(n, dtype=np.float64) for name in ("h", "g", "u", "ag", "au")}
    lib = _load()
    _run(lambda r0, r1: lib.q4k_fused_swiglu_oracle_into(
        _ptr(rg[r0:r1]), _ptr(ru[r0:r1]), _ptr(x), k, 0, r1 - r0,
        *(_ptr(out[nm][r0:r1]) for nm in ("h", "g", "u", "ag", "au"))), n, threads)
    return out


def gemv_residual(w: np.ndarray, x: np.ndarray, r: np.ndarray, threads: int = 1):
    """(y, A): y[n] = sum_k W[n,k] x[k] + r[n] (f64), A[n] = sum_k |W[n,k] x[k]| + |r[n]|."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    r = np.ascontiguousarray(r, dtype=np.float32).reshape(-1)
    k = x.size
    rows = _as_rows(w, k)
    n = rows.shape[0]
    if r.size != n:
        raise ValueError(f"residual has {r.size} entries for {n} rows")
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    lib = _load()
    _run(lambda r0, r1: lib.q4k_gemv_residual_oracle_into(_ptr(rows[r0:r1]), _ptr(x), _ptr(r[r0:r1]), k, 0, r1 - r0,
                                                          _ptr(y[r0:r1]), _ptr(a[r0:r1])), n, threads)
    return y, a


def gemv_multi(ws, x: np.ndarray, threads: int = 1):
    """[(y_j, A_j)]: one GEMV per matrix of ``ws``, all against the same x."""
    return [gemv(w, x, threads=threads) for w in ws]


def split_qg(y: np.ndarray, head_dim: int):
    """(q, gate): the per-head de-interleave of a q projection's output
    ("@simulatte/doppler 0.1.7 -> 0.1.8", kernels/split_qg.wgsl): the rows
    of head h are 2*head_dim apart, its first head_dim rows are q and the
    next head_dim the gate, so q[h*D + d] = y[h*2D + d] and
    gate[h*D + d] = y[h*2D + D + d] with D = head_dim."""
    y = np.asarray(y)
    n = y.shape[0]
    d2 = 2 * head_dim
    if head_dim <= 0 or n % d2 != 0:
        raise ValueError("the output length must be a multiple of 2 * head_dim")
    q = np.empty(n // 2, dtype=y.dtype)
    g = np.empty(n // 2, dtype=y.dtype)
    for h in range(n // d2):
        for d in range(head_dim):
            q[h * head_dim + d] = y[h * d2 + d]
            g[h * head_dim + d] = y[h * d2 + head_dim + d]
    return q, g


# ------------------------------------------------------------------- Q8_0
def _q8_rows(w: np.ndarray, k: int) -> np.ndarray:
    if k % Q8_0_BLOCK_WEIGHTS != 0:
        raise ValueError(f"k={k} is not a multiple of {Q8_0_BLOCK_WEIGHTS}")
    rb = (k // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES
    w = np.ascontiguousarray(w, dtype=np.uint8).reshape(-1)
    if rb == 0 or w.size % rb != 0:
        raise ValueError(f"{w.size} bytes is not a whole number of {rb}-byte rows")
    return w.reshape(-1, rb)


def q8_0_dequant_block(block34: bytes) -> np.ndarray:
    """The 32 f32 weights of one Q8_0 block."""
    buf = np.frombuffer(bytes(block34), dtype=np.uint8).copy()
    if buf.size != Q8_0_BLOCK_BYTES:
        raise ValueError("a Q8_0 block is 34 bytes")
    out = np.empty(Q8_0_BLOCK_WEIGHTS, dtype=np.float32)
    _load().q8_0_oracle_dequant_block(_ptr(buf), _ptr(out))
    return out


def q8_0_dequant(w: np.ndarray, k: int, threads: int = 1) -> np.ndarray:
    """A Q8_0 matrix as f32 [n, k]."""
    rows = _q8_rows(w, k)
    n = rows.shape[0]
    out = np.empty((n, k), dtype=np.float32)
    lib = _load()
    _run(lambda a, b: lib.q8_0_oracle_dequant_rows(_ptr(rows), k, a, b, _ptr(out[a:b])), n, threads)
    return out


def q8_0_gemv(w: np.ndarray, x: np.ndarray, threads: int = 1):
    """(y, A): y[n] = sum_k W[n,k] x[k] (f64) for a Q8_0 matrix, A[n] = sum_k |W[n,k] x[k]|."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    k = x.size
    rows = _q8_rows(w, k)
    n = rows.shape[0]
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    lib = _load()
    _run(lambda r0, r1: lib.q8_0_gemv_oracle_into(_ptr(rows[r0:r1]), _ptr(x), k, 0, r1 - r0,
                                                  _ptr(y[r0:r1]), _ptr(a[r0:r1])), n, threads)
    return y, a
