"""A second, independent Q4_K decoder used only to pin the oracle.

It is written from the bit positions of the super-block, not from the
oracle's byte/sub-block loops: the twelve scale bytes are read as one 96-bit
little-endian integer and each six-bit field is cut out by its bit offsets;
each weight's code is found from its own index.  Vectorised numpy, f32 with
the same three roundings (d*sc, dmin*m, dl*q - ml), each a separate numpy op
so nothing is fused.
"""

from __future__ import annotations

import numpy as np

# Bit offsets inside the 96-bit scale field, per sub-block j:
#   (low-part offset, low-part width, high-part offset or None)
# Scales of sub-blocks 0-3 sit whole at bits 8j..8j+5; mins at 32+8j.
# Sub-blocks 4-7 (i = j-4): low 4 bits of the scale at 64+8i, of the min at
# 68+8i; top 2 bits of the scale at 8i+6, of the min at 32+8i+6.
_SC_FIELDS = [(8 * j, 6, None) for j in range(4)] + [(64 + 8 * i, 4, 8 * i + 6) for i in range(4)]
_M_FIELDS = [(32 + 8 * j, 6, None) for j in range(4)] + [(68 + 8 * i, 4, 32 + 8 * i + 6) for i in range(4)]


def _bits(s96: np.ndarray, off: int, width: int) -> np.ndarray:
    # s96: [nb, 12] u8 ; extract `width` bits starting at bit `off` (width <= 8,
    # field never crosses... handle crossing generally via 16-bit window).
    byte = off // 8
    shift = off % 8
    lo = s96[:, byte].astype(np.uint32)
    hi = s96[:, byte + 1].astype(np.uint32) if byte + 1 < 12 else np.zeros_like(lo)
    return ((lo | (hi << 8)) >> shift) & ((1 << width) - 1)


def scales_mins(blocks: np.ndarray):
    """[nb,144] u8 -> (sc [nb,8], m [nb,8]) as int."""
    s96 = blocks[:, 4:16]
    sc = np.empty((blocks.shape[0], 8), dtype=np.int64)
    m = np.empty((blocks.shape[0], 8), dtype=np.int64)
    for j in range(8):
        for out, fields in ((sc, _SC_FIELDS), (m, _M_FIELDS)):
            off, width, top = fields[j]
            v = _bits(s96, off, width)
            if top is not None:
                v = v | (_bits(s96, top, 2) << 4)
            out[:, j] = v
    return sc, m


def codes(blocks: np.ndarray) -> np.ndarray:
    """[nb,144] u8 -> [nb,256] codes 0..15."""
    e = np.arange(256)
    byte_index = 16 + 32 * (e // 64) + (e % 32)
    shift = np.where((e % 64) >= 32, 4, 0)
    return (blocks[:, byte_index].astype(np.int64) >> shift) & 15


def dequant(blocks: np.ndarray) -> np.ndarray:
    """[nb,144] u8 -> [nb,256] f32 weights."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1, 144)
    d = blocks[:, 0:2].copy().view("<f2").astype(np.float32)[:, 0]
    dmin = blocks[:, 2:4].copy().view("<f2").astype(np.float32)[:, 0]
    sc, m = scales_mins(blocks)
    q = codes(blocks)
    sub = np.arange(256) // 32
    dl = d[:, None] * sc.astype(np.float32)  # [nb, 8] f32
    ml = dmin[:, None] * m.astype(np.float32)
    t = dl[:, sub] * q.astype(np.float32)
    return (t - ml[:, sub]).astype(np.float32)


def pack_scales(sc, m) -> bytes:
    """Inverse of the six-bit packing (eight scales, eight mins -> 12 bytes)."""
    s = [0] * 12
    for j in range(4):
        s[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return bytes(s)
