"""Reader for the hand-worked fixtures under tests/golden/."""

from __future__ import annotations

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_kv(name: str) -> dict[str, str]:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def single_block() -> dict:
    kv = read_kv("q4k_single_block.txt")
    d = int(kv["d_bits"], 16)
    dmin = int(kv["dmin_bits"], 16)
    scales = bytes(int(t, 16) for t in kv["scales_hex"].split())
    assert kv["qs"] == "range(128)"
    qs = bytes(range(128))
    block = bytes([d & 0xFF, d >> 8, dmin & 0xFF, dmin >> 8]) + scales + qs
    assert len(block) == 144
    scale_min = [tuple(int(v) for v in p.split(",")) for p in kv["scale_min"].split()]
    weights = {int(a): float(b) for a, b in (p.split(":") for p in kv["weights"].split())}
    return {
        "block": block,
        "scale_min": scale_min,
        "weights": weights,
        "subblock_sums": [float(v) for v in kv["subblock_sums"].split()],
        "y_ones": float(kv["y_ones"]),
        "a_ones": float(kv["a_ones"]),
        "y_alternating": float(kv["y_alternating"]),
        "y_index": float(kv["y_index"]),
    }


def q8_0_two_blocks() -> dict:
    kv = read_kv("q8_0_two_blocks.txt")
    d0 = int(kv["d0_bits"], 16)
    d1 = int(kv["d1_bits"], 16)
    q0 = [-128] + [e - 16 for e in range(1, 31)] + [127]
    q1 = [(e % 4) - 1 for e in range(32)]
    row = (bytes([d0 & 0xFF, d0 >> 8]) + bytes(v & 0xFF for v in q0)
           + bytes([d1 & 0xFF, d1 >> 8]) + bytes(v & 0xFF for v in q1))
    assert len(row) == 68
    return {
        "row": row,
        "weights": {int(a): float(b) for a, b in (p.split(":") for p in kv["weights"].split())},
        "y_ones": float(kv["y_ones"]),
        "a_ones": float(kv["a_ones"]),
        "y_alternating": float(kv["y_alternating"]),
        "y_index": float(kv["y_index"]),
    }
