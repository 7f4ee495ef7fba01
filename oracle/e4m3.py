"""E4M3 codec of the oracle (test infrastructure only).

The pages name one FP8 format for every tensor and stage, E4M3 ("How the
unified E4M3 format adds to DeepSeek-V3's efficiency", section "Fine-grained
quantization strategy"; "Advantages of using FP8 for GEMM operations in
DeepSeek-V3", item 6).  They do not say which E4M3 variant.  Reading taken:
the OCP 8-bit "E4M3FN" variant -- 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, subnormals at exponent field 0, no infinities, NaN only at
S.1111.111, largest finite magnitude 448.

Encoding reading: round to nearest, ties to the even code, and saturate any
magnitude at or above 448 to 448.  Negative values that round to zero keep
their sign (code 0x80).

The decoder is written from the format definition.  The encoder is written as
a search in the monotone table of the 127 finite non-negative magnitudes, so it
shares nothing with a bit-level conversion.
"""

import numpy as np

E4M3_MAX = 448.0
_NAN_MAG = 0x7F


def _decode_one(code: int) -> float:
    """Value of one E4M3 code from the format definition."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        # subnormal: m/8 * 2^(1-7)
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
# Finite non-negative magnitudes, codes 0x00..0x7E, strictly increasing.
_MAG = _TABLE[:_NAN_MAG].copy()
# Midpoint between consecutive magnitudes (exact in float64: each value has at
# most 4 significant bits).
_MID = (_MAG[:-1] + _MAG[1:]) * 0.5


def decode_table() -> np.ndarray:
    """float64[256]: the value of every code (NaN for 0x7F and 0xFF)."""
    return _TABLE.copy()


def decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def encode(y) -> np.ndarray:
    """Encode float32 values to E4M3 codes (RNE, saturating at 448).

    The magnitude is located in the table of finite magnitudes: the lower
    neighbour is the largest table entry not above it, and the value goes to
    the upper neighbour when it lies above their midpoint, or exactly on it
    and the lower neighbour's code is odd (ties to even).
    """
    y = np.asarray(y, dtype=np.float32)
    sign = np.signbit(y).astype(np.uint8)
    nan = np.isnan(y)
    v = np.abs(y).astype(np.float64)
    v = np.where(nan, 0.0, v)
    lo = np.searchsorted(_MAG, v, side="right") - 1
    lo = np.clip(lo, 0, _NAN_MAG - 1)
    below_top = lo < _NAN_MAG - 1
    mid = _MID[np.minimum(lo, _NAN_MAG - 2)]
    up = below_top & ((v > mid) | ((v == mid) & (lo % 2 == 1)))
    mag = (lo + up).astype(np.uint8)
    mag = np.where(v >= E4M3_MAX, np.uint8(0x7E), mag)
    mag = np.where(nan, np.uint8(_NAN_MAG), mag)
    return (mag | (sign << 7)).astype(np.uint8)
