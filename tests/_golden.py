"""Readers for the hand-derived fixtures under tests/golden/."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def e4m3_codes():
    """[(code, value_str)] from e4m3_codes.txt."""
    return [(int(a, 16), b) for a, b in (l.split()[:2] for l in _lines("e4m3_codes.txt"))]


def e4m3_rounding():
    """[(input_str, code)] from e4m3_rounding.txt."""
    out = []
    for l in _lines("e4m3_rounding.txt"):
        p = l.split()
        out.append((p[0], int(p[1], 16)))
    return out


def quant_tiles():
    """{name: (entries{idx: value_str}, scale_bits, codes{idx: code})}."""
    tiles, scales, codes = {}, {}, {}
    for l in _lines("quant_tiles_worked.txt"):
        p = l.split()
        kind, name, rest = p[0], p[1], p[2:]
        if kind == "tile":
            tiles[name] = {int(i): v for i, v in (e.split(":") for e in rest)}
        elif kind == "scale":
            scales[name] = int(rest[0], 16)
        elif kind == "codes":
            codes[name] = {int(i): int(c, 16) for i, c in (e.split(":") for e in rest)}
    return {k: (tiles[k], scales[k], codes[k]) for k in tiles}
