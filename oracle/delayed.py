"""Delayed (history-based) scaling of 1x128 activation tiles, the baseline the
pages compare online scaling against (test infrastructure only).

What the pages fix
------------------
"How online quantization in DeepSeek-V3 differs from delayed quantization",
items 2-4: delayed quantization takes its scaling factors from maxima seen in
earlier iterations, which it has to keep in a stored history; online
quantization takes them from the current values.  The pages give neither the
granularity nor the length of the history.

Readings taken
--------------
* The history holds the largest magnitude of each of the last ``H`` steps;
  the scale of step ``t`` comes from the maximum over steps ``t-H .. t-1``
  (the window), by the same rule as online scaling:
  ``s = RN32(a/448)``, ``r = RN32(448/a)``, ``q = E4M3_RNE_SAT(RN32(x*r))``
  with ``a = max(window maximum, 2^-64)``.
* Two granularities:
  - ``"tile"``: one history per 1x128 tile position (the online groups, so
    that only the timeliness of the scale differs).  Ring ``hist[H][KB][M]``;
    step ``u`` lives in slot ``u % H``; step ``t`` reads all ``H`` slots, then
    stores its own maxima in slot ``t % H``.
  - ``"tensor"``: one history for the whole tensor, the usual practice of
    earlier FP8 frameworks.  Ring ``hist[H + 2]``; step ``u`` lives in slot
    ``u % (H + 2)``; step ``t`` reads the ``H`` window slots, raises slot
    ``t % (H + 2)`` to the current tensor maximum and clears slot
    ``(t + 1) % (H + 2)`` (the slot the next step raises; it holds step
    ``t - H - 1``, outside every window still to come).
* A group whose window maximum is 0 (no history yet, e.g. the first step of
  a history that starts at zero) is scaled from its own current maximum,
  i.e. online.
* Values that the stale scale pushes past the E4M3 range saturate to +-448.
  ``saturated`` counts the values that saturation actually changes: those
  with ``|RN32(x*r)| > 464``, the midpoint between 448 and the next step of
  the binade (480), above which round-to-nearest would leave the format.
  (Online scaling puts a tile's maximum within 2^-14 of 448, which rounds to
  448 and is not counted.)  ``flushed`` counts non-zero values that round to
  a zero code.
"""

import numpy as np

from .e4m3 import encode
from .quant import TILE, bf16_bits_to_f32, tile_scale


def _tile_max(x):
    M, K = x.shape
    KB = K // TILE
    return np.max(np.abs(x).reshape(M, KB, TILE), axis=2).T.astype(np.float32)  # [KB][M]


def quant_act_1x128_delayed(x_bits, hist, step, mode):
    """One step of delayed scaling.

    x_bits: bf16 bits [M][K] (K % 128 == 0); hist: float32 ring (layout per
    ``mode`` above, not modified); step: t >= 0.
    Returns ``(q, s, hist_after, stats)``: codes uint8 [M][K]; scales float32
    [KB][M]; the ring after the step; ``stats`` = (saturated, flushed).
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    M, K = x.shape
    assert K % TILE == 0
    KB = K // TILE
    cur = _tile_max(x)
    hist = np.array(hist, dtype=np.float32, copy=True)
    if mode == "tile":
        H = hist.shape[0]
        assert hist.shape[1:] == (KB, M)
        window = np.max(hist, axis=0)
        hist[step % H] = cur
    elif mode == "tensor":
        H = hist.shape[0] - 2
        assert H >= 1
        slots = [(step - 1 - d) % (H + 2) for d in range(H)]
        window = np.full((KB, M), np.max(hist[slots]), dtype=np.float32)
        w = step % (H + 2)
        hist[w] = max(hist[w], np.max(cur))
        hist[(step + 1) % (H + 2)] = 0.0
    else:
        raise ValueError(mode)
    a = np.where(window > 0, window, cur)
    s, r = tile_scale(a)
    rr = np.repeat(r.T, TILE, axis=1)  # [M][K]
    y = np.multiply(x, rr, dtype=np.float32)
    q = encode(y)
    saturated = int(np.count_nonzero(np.abs(y) > np.float32(464.0)))
    flushed = int(np.count_nonzero((x != 0) & ((q & 0x7F) == 0)))
    return q, s, hist, (saturated, flushed)
