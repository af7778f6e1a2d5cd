"""The Python binding's host-side checks, without a GPU.

The library sees only pointers and sizes, so the binding is the one place
that can compare the tensors a caller passes with the sizes it hands over.
Each wrapper must refuse, before any library call, an output of the wrong
length, a residual of the wrong length, a weight tensor shorter than the rows
it is asked to read, and tensors on different devices.  A recording stand-in
for the loaded library shows that nothing reaches it."""

from __future__ import annotations

import re

import pytest
import torch

from q4_dequant_gemv_amd import q4k

K = 512
N = 8


class Recorder:
    """Stands in for the ctypes library: every attribute is a function that
    records its call."""

    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0

        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(q4k, "_lib", r)
    return r


def w_rows(n=N, k=K):
    return torch.zeros(n * (k // 256) * 144, dtype=torch.uint8)


def f32(*shape, device="cpu"):
    return torch.zeros(*shape, dtype=torch.float32, device=device)


CASES = {
    # wrapper call -> the message fragment of its ValueError
    "gemv short y": (lambda: q4k.gemv(w_rows(), f32(K), y=f32(N - 1)), "y has 7 elements"),
    "gemv long y": (lambda: q4k.gemv(w_rows(), f32(K), y=f32(N + 1)), "y has 9 elements"),
    "gemv n beyond w": (lambda: q4k.gemv(w_rows(), f32(K), y=f32(N + 2), n=N + 2), "w holds"),
    "gemv y on another device": (lambda: q4k.gemv(w_rows(), f32(K), y=f32(N, device="meta")), "y is on meta"),
    "gemv w on another device": (lambda: q4k.gemv(w_rows().to("meta"), f32(K), y=f32(N), n=N), "w is on meta"),
    "gemv_dt short y": (lambda: q4k.gemv_dt(w_rows(), f32(K), y=f32(N - 1)), "y has 7"),
    "residual short r": (lambda: q4k.gemv_residual(w_rows(), f32(K), f32(N - 1), y=f32(N)), "r has 7"),
    "residual short y": (lambda: q4k.gemv_residual(w_rows(), f32(K), f32(N), y=f32(N - 1)), "y has 7"),
    "residual r on another device": (lambda: q4k.gemv_residual(w_rows(), f32(K), f32(N, device="meta"), y=f32(N)),
                                     "r is on meta"),
    "batched short y": (lambda: q4k.gemv_batched(w_rows(), f32(3, K), y=f32(3, N - 1)), "y has 21"),
    "batched n beyond w": (lambda: q4k.gemv_batched(w_rows(), f32(3, K), y=f32(3, N + 1), n=N + 1), "w holds"),
    "batched_dt short y": (lambda: q4k.gemv_batched_dt(w_rows(), f32(3, K), y=f32(2, N)), "y has 16"),
    "batched_ws short y": (lambda: q4k.gemv_batched_ws(w_rows(), f32(3, K), None, y=f32(2, N)), "y has 16"),
    "batched_ws workspace elsewhere": (
        lambda: q4k.gemv_batched_ws(w_rows(), f32(3, K), torch.zeros(256, dtype=torch.uint8, device="meta"),
                                    y=f32(3, N)), "workspace is on meta"),
    "prefill short y": (lambda: q4k.prefill_gemm(w_rows(), torch.zeros(4, K, dtype=torch.float16), y=f32(4, N - 1)),
                        "y has 28"),
    "prefill_ws short y": (lambda: q4k.prefill_gemm_ws(w_rows(), torch.zeros(4, K, dtype=torch.float16), None,
                                                       y=f32(4, N - 1)), "y has 28"),
    "swiglu short h": (lambda: q4k.fused_swiglu(w_rows(), w_rows(), f32(K), h=f32(N - 1)), "h has 7"),
    "swiglu short up matrix": (lambda: q4k.fused_swiglu(w_rows(), w_rows(N - 1), f32(K), h=f32(N), n=N),
                               "w_up holds"),
    "dequant short out": (lambda: q4k.dequant(w_rows(), K, out=f32(N, K - 1)), "out has"),
    "dequant n beyond w": (lambda: q4k.dequant(w_rows(), K, out=f32(N + 1, K), n=N + 1), "w holds"),
    "q8_0 short y": (lambda: q4k.q8_0_gemv(torch.zeros(N * (K // 32) * 34, dtype=torch.uint8), f32(K),
                                           y=f32(N - 1)), "y has 7"),
    "q8_0 n beyond w": (lambda: q4k.q8_0_gemv(torch.zeros(N * (K // 32) * 34, dtype=torch.uint8), f32(K),
                                              y=f32(N + 1), n=N + 1), "w holds"),
    "multi short y": (lambda: q4k.gemv_multi([w_rows(), w_rows()], f32(K), ys=[f32(N), f32(N - 1)]), "ys[1] has 7"),
    "multi n beyond w": (lambda: q4k.gemv_multi([w_rows()], f32(K), ys=[f32(N + 1)], ns=[N + 1]), "ws[0] holds"),
    "multi short gate": (lambda: q4k.gemv_multi([w_rows()], f32(K), ys=[f32(N // 2)], gates=[f32(N // 2 - 1)],
                                                head_dims=[2]), "gates[0] has 3"),
    "split_qg short q": (lambda: q4k.gemv_split_qg(w_rows(), f32(K), 2, q=f32(N // 2 - 1)), "ys[0] has 3"),
    "negative n": (lambda: q4k.gemv(w_rows(), f32(K), y=f32(0), n=-1), "negative size"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_mismatch_raises_before_any_library_call(rec, name):
    call, fragment = CASES[name]
    with pytest.raises(ValueError, match=re.escape(fragment)):
        call()
    assert rec.calls == [], f"{name}: the library was called: {rec.calls}"


def test_matching_sizes_reach_only_the_device_check(rec):
    # with every size right the next refusal is that the tensors live on the
    # host; still nothing is called
    with pytest.raises(ValueError, match="must be a device tensor"):
        q4k.gemv(w_rows(), f32(K), y=f32(N))
    with pytest.raises(ValueError, match="must be a device tensor"):
        q4k.gemv_batched(w_rows(), f32(3, K), y=f32(3, N))
    assert rec.calls == []


def test_non_tensor_arguments_raise_type_error(rec):
    with pytest.raises(TypeError):
        q4k.gemv(w_rows(), [0.0] * K)
    with pytest.raises(TypeError):
        q4k.gemv_residual(w_rows(), f32(K), [0.0] * N, y=f32(N))
    assert rec.calls == []
