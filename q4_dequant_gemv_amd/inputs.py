"""Seeded synthetic inputs for the Q4_K path.

This module is the only code shared by the HIP path's tests/benchmark and the
CPU oracle.  It draws random bytes and numbers and lays them out in the
144-byte super-block format; it performs none of the method's arithmetic
(no scale/min unpacking, no nibble decoding, no dequantization, no dot).

Value distributions stand in for the Qwen3.5 Q4_K_M weights the pages
measure (issue #3346: size_variants.9b constants and the measured 0.8B
inventory), which are not available:
  * code bytes ``qs`` uniform 0..255 (every nibble uniform 0..15),
  * packed scale bytes uniform 0..255 (every six-bit scale and min uniform
    0..63, the 12-byte packing being a bijection on 96 bits),
  * ``d`` and ``dmin`` drawn uniform in [1e-3, 1e-2] in f64, then rounded to
    IEEE binary16 (round to nearest even),
  * activations f64 standard normal rounded to f32.
Streams are numpy PCG64 seeded by ``SeedSequence([seed, config_id, tensor_id])``;
within a weight tensor the draw order is qs, scales, d, dmin.
"""

from __future__ import annotations

import numpy as np

BLOCK_BYTES = 144
BLOCK_WEIGHTS = 256

# The shapes the pages give (issue #3346): Qwen3.5-0.8B measured tensors and
# the Qwen3.5-9B size variant.
SHAPES = {
    "square_1k": (1024, 1024),
    "q_proj_0p8b": (4096, 1024),
    "out_proj_0p8b": (1024, 2048),
    "lm_head_0p8b": (248320, 1024),
    "gate_9b": (12288, 4096),
    "up_9b": (12288, 4096),
    "down_9b": (4096, 12288),
    "lm_head_9b": (248320, 4096),
    # one GPU's share of the 9B decode matrices split eight ways: a
    # vocabulary (row) shard of the lm_head, a row shard of gate/up, and a
    # split-K shard of down (1536 columns: 6 super-blocks of each row)
    "lm_head_9b_shard8": (31040, 4096),
    "gate_9b_shard8": (1536, 4096),
    "down_9b_kshard8": (4096, 1536),
    # input projections of a Qwen3.5-0.8B linear-attention (GatedDeltaNet)
    # layer, all read against the same normed hidden state (the
    # hf_qwen35_linear_attn_debug.py trace: qkv is 6144 wide, 16 heads of 128;
    # z has one value per v channel, a and b one per v head)
    "gdn_qkv_0p8b": (6144, 1024),
    "gdn_z_0p8b": (2048, 1024),
    "gdn_a_0p8b": (16, 1024),
    "gdn_b_0p8b": (16, 1024),
}
GDN_PROJECTIONS_0P8B = ("gdn_qkv_0p8b", "gdn_z_0p8b", "gdn_a_0p8b", "gdn_b_0p8b")


def rng(config_id: int, tensor_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config_id, tensor_id])))


def row_bytes(k: int) -> int:
    if k % BLOCK_WEIGHTS != 0:
        raise ValueError(f"k={k} is not a multiple of {BLOCK_WEIGHTS}")
    return (k // BLOCK_WEIGHTS) * BLOCK_BYTES


def assemble_blocks(qs: np.ndarray, scales: np.ndarray, d: np.ndarray, dmin: np.ndarray) -> np.ndarray:
    """Lay fields out as 144-byte super-blocks: d | dmin | scales[12] | qs[128].

    ``qs`` [nb,128] u8, ``scales`` [nb,12] u8, ``d``/``dmin`` [nb] f16.
    Returns [nb, 144] u8.
    """
    nb = qs.shape[0]
    out = np.empty((nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d, dtype="<f2").view(np.uint8).reshape(nb, 2)
    out[:, 2:4] = np.ascontiguousarray(dmin, dtype="<f2").view(np.uint8).reshape(nb, 2)
    out[:, 4:16] = scales
    out[:, 16:144] = qs
    return out


def make_q4k(n: int, k: int, config_id: int = 0, tensor_id: int = 0, seed: int = 0,
             d_range=(1e-3, 1e-2)) -> np.ndarray:
    """A random Q4_K matrix of n rows by k columns as u8 [n, (k/256)*144]."""
    rb = row_bytes(k)
    nb = n * (k // BLOCK_WEIGHTS)
    g = rng(config_id, tensor_id, seed)
    qs = g.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    scales = g.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    d = g.uniform(d_range[0], d_range[1], size=nb).astype(np.float16)
    dmin = g.uniform(d_range[0], d_range[1], size=nb).astype(np.float16)
    return assemble_blocks(qs, scales, d, dmin).reshape(n, rb)


Q8_0_BLOCK_BYTES = 34
Q8_0_BLOCK_WEIGHTS = 32


def q8_0_row_bytes(k: int) -> int:
    if k % Q8_0_BLOCK_WEIGHTS != 0:
        raise ValueError(f"k={k} is not a multiple of {Q8_0_BLOCK_WEIGHTS}")
    return (k // Q8_0_BLOCK_WEIGHTS) * Q8_0_BLOCK_BYTES


def assemble_q8_0(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Lay fields out as 34-byte Q8_0 blocks: d (f16) | q[32] (int8).  Returns [nb, 34] u8."""
    nb = q.shape[0]
    out = np.empty((nb, Q8_0_BLOCK_BYTES), dtype=np.uint8)
    out[:, 0:2] = np.ascontiguousarray(d, dtype="<f2").view(np.uint8).reshape(nb, 2)
    out[:, 2:] = np.ascontiguousarray(q, dtype=np.int8).view(np.uint8)
    return out


def make_q8_0(n: int, k: int, config_id: int = 0, tensor_id: int = 0, seed: int = 0,
              d_range=(1e-4, 1e-3)) -> np.ndarray:
    """A random Q8_0 matrix of n rows by k columns as u8 [n, (k/32)*34]: codes
    uniform in [-127, 127] (a symmetric quantizer's range), d uniform in
    d_range rounded to f16.  Draw order: codes, then d."""
    rb = q8_0_row_bytes(k)
    nb = n * (k // Q8_0_BLOCK_WEIGHTS)
    g = rng(config_id, tensor_id, seed)
    q = g.integers(-127, 128, size=(nb, Q8_0_BLOCK_WEIGHTS), dtype=np.int8)
    d = g.uniform(d_range[0], d_range[1], size=nb).astype(np.float16)
    return assemble_q8_0(q, d).reshape(n, rb)


def make_x(m: int, k: int, config_id: int = 0, tensor_id: int = 100, seed: int = 0) -> np.ndarray:
    """Activations f32 [m, k], standard normal."""
    g = rng(config_id, tensor_id, seed)
    return g.standard_normal(size=(m, k)).astype(np.float32)
