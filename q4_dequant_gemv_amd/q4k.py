"""Python binding of libq4k.so (C ABI in include/q4k.h).

Argument marshalling only: tensors become device pointers, the current torch
HIP stream becomes the ``stream`` argument, and any status other than
``Q4K_OK`` raises ``Q4KError``.  Every step of the computation runs in the
library's HIP kernels; there is no CPU path.  The library must have been built
(``python -m q4_dequant_gemv_amd.build`` or ``__graft_entry__.build()``); if it
is missing, loading raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq4k.so")

BLOCK_BYTES = 144
BLOCK_WEIGHTS = 256

STATUS = {0: "Q4K_OK", 1: "Q4K_ERR_INVALID_ARG", 2: "Q4K_ERR_UNSUPPORTED_SHAPE", 3: "Q4K_ERR_MISALIGNED",
          4: "Q4K_ERR_LAUNCH"}

# exported symbols, in the order include/q4k.h declares them
EXPORTS = ("q4k_gemv", "q4k_gemv_dt", "q4k_gemv_residual", "q4k_gemv_multi", "q4k_q8_0_gemv", "q4k_gemv_batched",
           "q4k_gemv_batched_dt", "q4k_gemv_batched_noalloc", "q4k_prefill_gemm", "q4k_gemv_batched_workspace_size",
           "q4k_gemv_batched_ws",
           "q4k_prefill_workspace_size", "q4k_prefill_gemm_ws", "q4k_fused_swiglu", "q4k_dequant",
           "q4k_status_string", "q4k_abi_version")

# alignment a workspace passed to the *_ws calls must have
WORKSPACE_ALIGN = 256

# q4k_dtype
F32, F16 = 0, 1

Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32

# largest number of matrices in one gemv_multi call (Q4K_MAX_MULTI)
MAX_MULTI = 8


class GemvItem(ctypes.Structure):
    """q4k_gemv_item: one matrix of a gemv_multi call."""

    _fields_ = [("w", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("y_gate", ctypes.c_void_p), ("head_dim", ctypes.c_int64)]


class Q4KError(RuntimeError):
    def __init__(self, status: int, call: str, detail: str):
        super().__init__(f"{call}: {STATUS.get(status, status)} ({detail})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libq4k.so with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m q4_dequant_gemv_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.q4k_gemv.argtypes = [p, p, p, i64, i64, p]
        L.q4k_gemv_residual.argtypes = [p, p, p, p, i64, i64, p]
        L.q4k_gemv_multi.argtypes = [ctypes.POINTER(GemvItem), ctypes.c_int, p, i64, p]
        L.q4k_q8_0_gemv.argtypes = [p, p, p, i64, i64, p]
        L.q4k_gemv_dt.argtypes = [p, p, ctypes.c_int, p, ctypes.c_int, i64, i64, p]
        L.q4k_gemv_batched_dt.argtypes = [p, p, ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p]
        L.q4k_gemv_batched_noalloc.argtypes = [p, p, ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p]
        L.q4k_prefill_gemm.argtypes = [p, p, p, ctypes.c_int, i64, i64, i64, p]
        L.q4k_gemv_batched.argtypes = [p, p, p, i64, i64, i64, p]
        pi64 = ctypes.POINTER(i64)
        L.q4k_gemv_batched_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, pi64]
        L.q4k_gemv_batched_ws.argtypes = [p, p, ctypes.c_int, p, ctypes.c_int, i64, i64, i64, p, i64, p]
        L.q4k_prefill_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, pi64]
        L.q4k_prefill_gemm_ws.argtypes = [p, p, p, ctypes.c_int, i64, i64, i64, p, i64, p]
        L.q4k_fused_swiglu.argtypes = [p, p, p, p, i64, i64, p]
        L.q4k_dequant.argtypes = [p, p, i64, i64, p]
        for f in (L.q4k_gemv, L.q4k_gemv_dt, L.q4k_gemv_residual, L.q4k_gemv_multi, L.q4k_q8_0_gemv,
                  L.q4k_gemv_batched, L.q4k_gemv_batched_dt, L.q4k_gemv_batched_noalloc, L.q4k_prefill_gemm,
                  L.q4k_fused_swiglu, L.q4k_dequant):
            f.restype = st
        L.q4k_status_string.argtypes = [st]
        L.q4k_status_string.restype = ctypes.c_char_p
        L.q4k_abi_version.argtypes = []
        L.q4k_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().q4k_status_string(status).decode()


def _check(status: int, call: str) -> None:
    if status != 0:
        raise Q4KError(status, call, status_string(status))


def _stream(stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name, dtype):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def rows_of(w, k: int) -> int:
    if k % BLOCK_WEIGHTS != 0:
        raise ValueError(f"k={k} is not a multiple of {BLOCK_WEIGHTS}")
    rb = (k // BLOCK_WEIGHTS) * BLOCK_BYTES
    if rb == 0:
        raise ValueError("k must be positive to infer the row count; pass n")
    if w.numel() % rb != 0:
        raise ValueError(f"weight tensor of {w.numel()} bytes is not a whole number of {rb}-byte rows")
    return w.numel() // rb


def _tensor(t, name):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    return t


def _sizes(device, weights=(), exact=()):
    """Host-side size and placement checks made before anything reaches the
    library, which sees only pointers: every tensor on ``device``; each
    ``(w, name, bytes)`` of ``weights`` holds at least ``bytes`` bytes; each
    ``(t, name, count)`` of ``exact`` has exactly ``count`` elements.  A
    mismatch raises ValueError and nothing is launched."""
    for t, name, need in weights:
        _tensor(t, name)
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the activations on {device}")
        if t.numel() < need:
            raise ValueError(f"{name} holds {t.numel()} bytes; the call reads {need}")
    for t, name, count in exact:
        _tensor(t, name)
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the activations on {device}")
        if t.numel() != count:
            raise ValueError(f"{name} has {t.numel()} elements; the call needs {count}")


def _q4k_bytes(n: int, k: int) -> int:
    if n < 0 or k < 0:
        raise ValueError(f"negative size (n={n}, k={k})")
    return n * (k // BLOCK_WEIGHTS) * BLOCK_BYTES


def gemv(w, x, y=None, n: int | None = None, stream=None):
    """y[r] = sum_c W[r,c] x[c] for a Q4_K matrix ``w`` (uint8) and f32 ``x`` [k]."""
    import torch

    k = _tensor(x, "x").numel()
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(y, "y", n)])
    _check(lib().q4k_gemv(_dev(w, "w", torch.uint8), _dev(x, "x", torch.float32), _dev(y, "y", torch.float32),
                          n, k, _stream(stream)), "q4k_gemv")
    return y


def _dtype_code(t, name):
    import torch

    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    raise TypeError(f"{name} must be float32 or float16 (got {t.dtype})")


def _dev_any(t, name):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def gemv_dt(w, x, y=None, n: int | None = None, out_dtype=None, stream=None):
    """``gemv`` with f16 or f32 ``x`` and ``y`` (the tensors' dtypes say which)."""
    import torch

    k = _tensor(x, "x").numel()
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty(n, dtype=out_dtype or x.dtype, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(y, "y", n)])
    _check(lib().q4k_gemv_dt(_dev(w, "w", torch.uint8), _dev_any(x, "x"), _dtype_code(x, "x"), _dev_any(y, "y"),
                             _dtype_code(y, "y"), n, k, _stream(stream)), "q4k_gemv_dt")
    return y


def gemv_batched_dt(w, x, y=None, n: int | None = None, out_dtype=None, stream=None):
    """``gemv_batched`` with f16 or f32 ``x`` [m, k] and ``y`` [m, n]."""
    import torch

    if _tensor(x, "x").dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype or x.dtype, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(y, "y", m * n)])
    _check(lib().q4k_gemv_batched_dt(_dev(w, "w", torch.uint8), _dev_any(x, "x"), _dtype_code(x, "x"),
                                     _dev_any(y, "y"), _dtype_code(y, "y"), m, n, k, _stream(stream)),
           "q4k_gemv_batched_dt")
    return y


# bytes of the per-GPU scratch array of gemv_batched_noalloc (Q4K_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 16 << 20


def gemv_batched_noalloc(w, x, y=None, n: int | None = None, out_dtype=None, stream=None):
    """``gemv_batched_dt`` with its scratch in the library's per-GPU array:
    the library allocates nothing (``y`` must be given to allocate nothing at
    all on this side either)."""
    import torch

    if _tensor(x, "x").dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype or x.dtype, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(y, "y", m * n)])
    _check(lib().q4k_gemv_batched_noalloc(_dev(w, "w", torch.uint8), _dev_any(x, "x"), _dtype_code(x, "x"),
                                          _dev_any(y, "y"), _dtype_code(y, "y"), m, n, k, _stream(stream)),
           "q4k_gemv_batched_noalloc")
    return y


def prefill_gemm(w, x, y=None, n: int | None = None, out_dtype=None, stream=None):
    """y[t, r] = sum_c W[r,c] x[t,c] for f16 ``x`` [m, k] (prefill sizes); ``y`` f32 or f16 [m, n]."""
    import torch

    if _tensor(x, "x").dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype or torch.float32, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(y, "y", m * n)])
    _check(lib().q4k_prefill_gemm(_dev(w, "w", torch.uint8), _dev(x, "x", torch.float16), _dev_any(y, "y"),
                                  _dtype_code(y, "y"), m, n, k, _stream(stream)), "q4k_prefill_gemm")
    return y


def _code_of(dtype, name):
    import torch

    if dtype == torch.float32:
        return F32
    if dtype == torch.float16:
        return F16
    raise TypeError(f"{name} must be float32 or float16 (got {dtype})")


def gemv_batched_workspace_size(m: int, n: int, k: int, x_dtype=None, out_dtype=None) -> int:
    """Bytes of workspace ``gemv_batched_ws`` needs on the current device (0: none)."""
    import torch

    out = ctypes.c_int64(-1)
    _check(lib().q4k_gemv_batched_workspace_size(_code_of(x_dtype or torch.float32, "x_dtype"),
                                                 _code_of(out_dtype or torch.float32, "out_dtype"), m, n, k,
                                                 ctypes.byref(out)), "q4k_gemv_batched_workspace_size")
    return out.value


def prefill_workspace_size(m: int, n: int, k: int, out_dtype=None) -> int:
    """Bytes of workspace ``prefill_gemm_ws`` needs on the current device (0: none)."""
    import torch

    out = ctypes.c_int64(-1)
    _check(lib().q4k_prefill_workspace_size(_code_of(out_dtype or torch.float32, "out_dtype"), m, n, k,
                                            ctypes.byref(out)), "q4k_prefill_workspace_size")
    return out.value


def _workspace(t):
    """(pointer, bytes) of a uint8 device workspace tensor, or (NULL, 0)."""
    import torch

    if t is None:
        return ctypes.c_void_p(0), 0
    return _dev(t, "workspace", torch.uint8), t.numel()


def gemv_batched_ws(w, x, workspace, y=None, n: int | None = None, out_dtype=None, stream=None):
    """``gemv_batched_dt`` with scratch taken from ``workspace`` (uint8, 256-byte aligned)."""
    import torch

    if _tensor(x, "x").dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype or x.dtype, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))] + ([] if workspace is None else [(workspace, "workspace", 0)]),
           [(y, "y", m * n)])
    wp, wb = _workspace(workspace)
    _check(lib().q4k_gemv_batched_ws(_dev(w, "w", torch.uint8), _dev_any(x, "x"), _dtype_code(x, "x"),
                                     _dev_any(y, "y"), _dtype_code(y, "y"), m, n, k, wp, wb, _stream(stream)),
           "q4k_gemv_batched_ws")
    return y


def prefill_gemm_ws(w, x, workspace, y=None, n: int | None = None, out_dtype=None, stream=None):
    """``prefill_gemm`` with scratch taken from ``workspace`` (uint8, 256-byte aligned)."""
    import torch

    if _tensor(x, "x").dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype or torch.float32, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))] + ([] if workspace is None else [(workspace, "workspace", 0)]),
           [(y, "y", m * n)])
    wp, wb = _workspace(workspace)
    _check(lib().q4k_prefill_gemm_ws(_dev(w, "w", torch.uint8), _dev(x, "x", torch.float16), _dev_any(y, "y"),
                                     _dtype_code(y, "y"), m, n, k, wp, wb, _stream(stream)), "q4k_prefill_gemm_ws")
    return y


def gemv_residual(w, x, r, y=None, n: int | None = None, stream=None):
    """y[i] = sum_c W[i,c] x[c] + r[i]; ``y`` may be ``r`` itself (in-place residual add)."""
    import torch

    k = _tensor(x, "x").numel()
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(r, "r", n), (y, "y", n)])
    _check(lib().q4k_gemv_residual(_dev(w, "w", torch.uint8), _dev(x, "x", torch.float32),
                                   _dev(r, "r", torch.float32), _dev(y, "y", torch.float32), n, k, _stream(stream)),
           "q4k_gemv_residual")
    return y


def gemv_multi(ws, x, ys=None, ns=None, gates=None, head_dims=None, stream=None):
    """ys[j][i] = sum_c W_j[i,c] x[c] for up to MAX_MULTI matrices sharing ``x``, in one launch.

    ``gates[j]`` (a tensor, or None) with ``head_dims[j]`` de-interleaves matrix
    j's output per head: its q rows go to ``ys[j]`` and its gate rows to
    ``gates[j]`` (n/2 each)."""
    import torch

    k = _tensor(x, "x").numel()
    ws = list(ws)
    ns = [rows_of(w, k) for w in ws] if ns is None else list(ns)
    gates = [None] * len(ws) if gates is None else list(gates)
    head_dims = [0] * len(ws) if head_dims is None else list(head_dims)
    if ys is None:
        ys = [torch.empty(n // 2 if g is not None else n, dtype=torch.float32, device=x.device)
              for n, g in zip(ns, gates)]
    ys = list(ys)
    if not (len(ws) == len(ys) == len(ns) == len(gates) == len(head_dims)):
        raise ValueError("ws, ys, ns, gates and head_dims must have the same length")
    for i, (w, y, n, g) in enumerate(zip(ws, ys, ns, gates)):
        ny = n // 2 if g is not None else n
        outs = [(y, f"ys[{i}]", ny)] + ([(g, f"gates[{i}]", ny)] if g is not None else [])
        _sizes(x.device, [(w, f"ws[{i}]", _q4k_bytes(n, k))], outs)
    items = (GemvItem * max(len(ws), 1))()
    for i, (w, y, n, g, hd) in enumerate(zip(ws, ys, ns, gates, head_dims)):
        items[i].w = _dev(w, f"ws[{i}]", torch.uint8).value
        items[i].y = _dev(y, f"ys[{i}]", torch.float32).value
        items[i].n = n
        items[i].y_gate = _dev(g, f"gates[{i}]", torch.float32).value if g is not None else None
        items[i].head_dim = hd
    _check(lib().q4k_gemv_multi(items, len(ws), _dev(x, "x", torch.float32), k, _stream(stream)), "q4k_gemv_multi")
    return ys


def gemv_split_qg(w, x, head_dim: int, q=None, g=None, n: int | None = None, stream=None):
    """The q projection of an attention-output-gate model with its output
    de-interleaved per head as it is stored: returns (q, gate), n/2 each."""
    import torch

    k = x.numel()
    n = rows_of(w, k) if n is None else n
    if q is None:
        q = torch.empty(n // 2, dtype=torch.float32, device=x.device)
    if g is None:
        g = torch.empty(n // 2, dtype=torch.float32, device=x.device)
    gemv_multi([w], x, ys=[q], ns=[n], gates=[g], head_dims=[head_dim], stream=stream)
    return q, g


def q8_0_rows_of(w, k: int) -> int:
    if k % Q8_0_BLOCK_WEIGHTS != 0:
        raise ValueError(f"k={k} is not a multiple of {Q8_0_BLOCK_WEIGHTS}")
    rb = (k // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES
    if rb == 0:
        raise ValueError("k must be positive to infer the row count; pass n")
    if w.numel() % rb != 0:
        raise ValueError(f"weight tensor of {w.numel()} bytes is not a whole number of {rb}-byte rows")
    return w.numel() // rb


def q8_0_gemv(w, x, y=None, n: int | None = None, stream=None):
    """y[r] = sum_c W[r,c] x[c] for a Q8_0 matrix ``w`` (uint8) and f32 ``x`` [k]."""
    import torch

    k = _tensor(x, "x").numel()
    n = q8_0_rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty(n, dtype=torch.float32, device=x.device)
    if n < 0:
        raise ValueError(f"negative size (n={n})")
    _sizes(x.device, [(w, "w", n * (k // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES)], [(y, "y", n)])
    _check(lib().q4k_q8_0_gemv(_dev(w, "w", torch.uint8), _dev(x, "x", torch.float32), _dev(y, "y", torch.float32),
                               n, k, _stream(stream)), "q4k_q8_0_gemv")
    return y


def gemv_batched(w, x, y=None, n: int | None = None, stream=None):
    """y[t, r] = sum_c W[r,c] x[t,c]; ``x`` f32 [m, k] -> ``y`` f32 [m, n]."""
    import torch

    if _tensor(x, "x").dim() != 2:
        raise ValueError("x must be [m, k]")
    m, k = x.shape
    n = rows_of(w, k) if n is None else n
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _sizes(x.device, [(w, "w", _q4k_bytes(n, k))], [(y, "y", m * n)])
    _check(lib().q4k_gemv_batched(_dev(w, "w", torch.uint8), _dev(x, "x", torch.float32),
                                  _dev(y, "y", torch.float32), m, n, k, _stream(stream)), "q4k_gemv_batched")
    return y


def fused_swiglu(w_gate, w_up, x, h=None, n: int | None = None, stream=None):
    """h[r] = silu((W_gate x)[r]) * (W_up x)[r]."""
    import torch

    k = _tensor(x, "x").numel()
    n = rows_of(w_gate, k) if n is None else n
    if h is None:
        h = torch.empty(n, dtype=torch.float32, device=x.device)
    _sizes(x.device, [(w_gate, "w_gate", _q4k_bytes(n, k)), (w_up, "w_up", _q4k_bytes(n, k))], [(h, "h", n)])
    _check(lib().q4k_fused_swiglu(_dev(w_gate, "w_gate", torch.uint8), _dev(w_up, "w_up", torch.uint8),
                                  _dev(x, "x", torch.float32), _dev(h, "h", torch.float32), n, k,
                                  _stream(stream)), "q4k_fused_swiglu")
    return h


def dequant(w, k: int, out=None, n: int | None = None, stream=None):
    """W as dense f32 [n, k], bit-exact."""
    import torch

    n = rows_of(_tensor(w, "w"), k) if n is None else n
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _sizes(w.device, [(w, "w", _q4k_bytes(n, k))], [(out, "out", n * k)])
    _check(lib().q4k_dequant(_dev(w, "w", torch.uint8), _dev(out, "out", torch.float32), n, k, _stream(stream)),
           "q4k_dequant")
    return out
