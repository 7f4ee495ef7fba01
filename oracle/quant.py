"""Online tile/block quantizers of the oracle (test infrastructure only).

What the pages fix
------------------
* "How online quantization in DeepSeek-V3 differs from delayed quantization",
  items 1-3: the scale of each 1x128 activation tile and each 128x128 weight
  block is computed from that tile's or block's own current values, every
  time, with no stored history of maxima.
* "How the unified E4M3 format adds to DeepSeek-V3's efficiency", sections
  "Fine-grained quantization strategy" and "Dynamic scaling and online
  quantization": the groups are 1x128 for activations and 128x128 for
  weights; each group's scale is chosen so that its values use the
  representable E4M3 values rather than bunching into a narrow range.

Readings taken where the pages are silent
-----------------------------------------
* Scale: the group's largest magnitude ``amax`` is mapped to the top of the
  E4M3 range, ``s = RN32(a / 448)`` stored as float32, with
  ``a = max(amax, 2^-64)`` so that an all-zero or tiny group still has a
  finite reciprocal.
* Quantize by multiplying with the reciprocal ``r = RN32(448 / a)``, computed
  once per group (one float32 rounding), then ``y = RN32(x * r)`` and
  ``q = E4M3(y)`` with round-to-nearest-even and saturation.
* A group at the edge of a tensor (fewer than 128 valid columns or rows) takes
  its ``amax`` over its valid elements only.

Layouts returned (conceptual, dense):
* activation: ``q`` uint8 [M][K], ``s`` float32 [ceil(K/128)][M]
  (scale of row m, tile kb at ``s[kb, m]``);
* weight: ``q`` uint8 [N][K], ``s`` float32 [ceil(N/128)][ceil(K/128)].
"""

import numpy as np

from .e4m3 import E4M3_MAX, encode

TILE = 128
SCALE_FLOOR = np.float32(2.0 ** -64)
_F448 = np.float32(E4M3_MAX)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen raw bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def tile_scale(amax):
    """Scale and reciprocal of a group from its largest magnitude.

    Returns ``(s, r)`` as float32 with ``a = max(amax, 2^-64)``,
    ``s = RN32(a / 448)`` and ``r = RN32(448 / a)`` (IEEE float32 division).
    """
    a = np.maximum(np.asarray(amax, dtype=np.float32), SCALE_FLOOR)
    with np.errstate(over="raise", divide="raise", invalid="ignore"):
        s = np.divide(a, _F448, dtype=np.float32)
        r = np.divide(_F448, a, dtype=np.float32)
    return s, r


def _quantize_group(x, r):
    """Codes of float32 values ``x`` scaled by float32 ``r`` (broadcast)."""
    y = np.multiply(x, r, dtype=np.float32)
    return encode(y)


def quant_rows_1x128(x):
    """Quantize float32 values [M][K] per 1x128 tile along each row.

    The steps of the online activation quantization (the pages' 1x128 tile
    rule) applied to float32 input: this is how a GEMM's FP32 output becomes
    the next GEMM's E4M3 input.  Returns ``(q, s)``: ``q`` uint8 [M][K];
    ``s`` float32 [KB][M] with ``KB = ceil(K/128)``.
    """
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    KB = -(-K // TILE)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((KB, M), dtype=np.float32)
    for kb in range(KB):
        k0, k1 = kb * TILE, min(K, (kb + 1) * TILE)
        t = x[:, k0:k1]
        amax = np.max(np.abs(t), axis=1)
        sk, rk = tile_scale(amax)
        q[:, k0:k1] = _quantize_group(t, rk[:, None])
        s[kb] = sk
    return q, s


def quant_act_1x128(x_bits, row_chunk: int = 2048):
    """Quantize bf16 activations [M][K] per 1x128 tile.

    The bf16 values are widened to float32 exactly, then quantized as
    ``quant_rows_1x128``.  Returns ``(q, s)``: ``q`` uint8 [M][K]; ``s``
    float32 [KB][M] with ``KB = ceil(K/128)``.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    KB = -(-K // TILE)
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((KB, M), dtype=np.float32)
    for m0 in range(0, M, row_chunk):
        m1 = min(M, m0 + row_chunk)
        q[m0:m1], s[:, m0:m1] = quant_rows_1x128(bf16_bits_to_f32(x_bits[m0:m1]))
    return q, s


def quant_w_128x128(w_bits, bands=None):
    """Quantize bf16 weights [N][K] per 128x128 block.

    Returns ``(q, s)``: ``q`` uint8 [N][K]; ``s`` float32 [NB][KB] with
    ``NB = ceil(N/128)`` and ``KB = ceil(K/128)``.

    ``bands`` optionally restricts the work to some 128-row bands (a list of
    ``nb``); rows of other bands are left as 0 in ``q`` and NaN in ``s``.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    N, K = w_bits.shape
    NB, KB = -(-N // TILE), -(-K // TILE)
    q = np.zeros((N, K), dtype=np.uint8)
    s = np.full((NB, KB), np.nan, dtype=np.float32)
    for nb in (range(NB) if bands is None else bands):
        n0, n1 = nb * TILE, min(N, (nb + 1) * TILE)
        x = bf16_bits_to_f32(w_bits[n0:n1])
        for kb in range(KB):
            k0, k1 = kb * TILE, min(K, (kb + 1) * TILE)
            blk = x[:, k0:k1]
            amax = np.max(np.abs(blk))
            sk, rk = tile_scale(amax)
            q[n0:n1, k0:k1] = _quantize_group(blk, rk)
            s[nb, kb] = sk
    return q, s
