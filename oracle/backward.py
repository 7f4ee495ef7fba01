"""Backward-pass operands and GEMMs in the same E4M3 format (test
infrastructure only).

What the pages fix
------------------
"How the unified E4M3 format adds to DeepSeek-V3's efficiency", section
"Fine-grained quantization strategy": E4M3 is used in every stage of training,
the backward pass included, where earlier frameworks switched to E5M2; the
fine-grained grouping is what makes that possible.  The pages give no group
orientation for the backward GEMMs.

Reading taken: every GEMM groups its operands 128-wide along its own
contraction dimension, as the forward GEMM does.  For a linear layer
Y = X . W^T (X [M][K], W [N][K]) with output gradient dY [M][N]:

* data gradient  dX [M][K] = dY . W: contraction over N.  dY is quantized
  per 1x128 tile along N (the activation rule); W keeps its 128x128 blocks,
  whose codes and scales are simply read transposed (W^T [K][N], block
  scales transposed).
* weight gradient dW [N][K] = dY^T . X: contraction over the M tokens.  Both
  dY and X are quantized in groups of 128 consecutive tokens per column
  (1x128 tiles of their transposes), so both operands carry one scale per
  row per 128-token group:
      dW[n, k] = sum_mb S_dY[mb, n] * S_X[mb, k] * sum_{m in mb} dec(QdY^T[n, m]) dec(QX^T[k, m])
"""

import numpy as np

from .e4m3 import decode_table
from .gemm import block_gemm
from .quant import TILE, quant_act_1x128, quant_w_128x128

_DEC = decode_table()


def quant_w_128x128_t(w_bits):
    """Weight codes and block scales, plus their transposes for dX = dY . W.

    Returns ``(q, s, qt, st)``: ``q`` [N][K], ``s`` [N/128][K/128] as
    ``quant_w_128x128``; ``qt = q^T`` [K][N]; ``st = s^T`` [K/128][N/128].
    """
    q, s = quant_w_128x128(w_bits)
    return q, s, np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def quant_act_128x1_t(x_bits):
    """Quantize bf16 [M][N] in groups of 128 consecutive rows per column.

    The groups are the 1x128 tiles of the transpose, so this is the
    activation quantizer applied to x^T.  Returns ``(qt, st)``: codes of x^T
    uint8 [N][M]; scales float32 [M/128][N] (``st[mb, n]``).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    return quant_act_1x128(np.ascontiguousarray(x_bits.T))


def block_gemm_rowscaled(qa, sa, qb, sb):
    """C = A . B^T with one scale per row per 128-K group on both operands.

    qa uint8 [M][K], sa float32 [K/128][M]; qb uint8 [N][K], sb float32
    [K/128][N].  C[m, n] = sum_kb sa[kb, m] * sb[kb, n] * P[m, n, kb], with P
    exact in float64 (as in ``block_gemm``).  Returns ``(C, B)`` float64
    [M][N]; ``B`` is the tolerance basis sum_kb sa sb sum_k |a b|.
    """
    qa = np.asarray(qa, dtype=np.uint8)
    qb = np.asarray(qb, dtype=np.uint8)
    M, K = qa.shape
    N, K2 = qb.shape
    assert K == K2 and K % TILE == 0
    C = np.zeros((M, N), dtype=np.float64)
    B = np.zeros((M, N), dtype=np.float64)
    for kb in range(K // TILE):
        k0 = kb * TILE
        a = _DEC[qa[:, k0:k0 + TILE]]
        b = _DEC[qb[:, k0:k0 + TILE]]
        scale = (np.asarray(sa[kb], dtype=np.float64)[:, None]
                 * np.asarray(sb[kb], dtype=np.float64)[None, :])
        C += scale * (a @ b.T)
        B += scale * (np.abs(a) @ np.abs(b).T)
    return C, B


def dgrad(dy_bits, w_bits):
    """dX = dY . W for bf16 dY [M][N] and W [N][K]: dY quantized per 1x128
    tile along N, W per 128x128 block read transposed.  Returns
    ``(qdy, sdy, qt, st, C, B)``."""
    qdy, sdy = quant_act_1x128(dy_bits)
    _, _, qt, st = quant_w_128x128_t(w_bits)
    C, B = block_gemm(qdy, sdy, qt, st)
    return qdy, sdy, qt, st, C, B


def wgrad(dy_bits, x_bits):
    """dW = dY^T . X for bf16 dY [M][N] and X [M][K], both quantized in
    128-token groups.  Returns ``(qdyt, sdyt, qxt, sxt, C, B)``."""
    qdyt, sdyt = quant_act_128x1_t(dy_bits)
    qxt, sxt = quant_act_128x1_t(x_bits)
    C, B = block_gemm_rowscaled(qdyt, sdyt, qxt, sxt)
    return qdyt, sdyt, qxt, sxt, C, B


def kgrouped_gemm_rowscaled(qa, sa, qb, sb, offsets):
    """MoE weight gradients in one call: for every expert g,
    C[g] = A[:, t0:t1] . B[:, t0:t1]^T over its token columns
    [t0, t1) = [offsets[g], offsets[g+1]) (multiples of 128: each expert's
    tokens padded with zero rows), with per-row scales on both operands as
    ``block_gemm_rowscaled``.  qa [M][T], sa [T/128][M]; qb [N][T],
    sb [T/128][N].  An expert without tokens gets C[g] = 0.
    Returns ``(C, B)`` float64 [G][M][N].
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    assert np.all(offsets % TILE == 0)
    G = len(offsets) - 1
    M, N = qa.shape[0], qb.shape[0]
    C = np.zeros((G, M, N))
    B = np.zeros((G, M, N))
    for g in range(G):
        t0, t1 = int(offsets[g]), int(offsets[g + 1])
        if t1 == t0:
            continue
        C[g], B[g] = block_gemm_rowscaled(qa[:, t0:t1], np.asarray(sa)[t0 // TILE:t1 // TILE],
                                          qb[:, t0:t1], np.asarray(sb)[t0 // TILE:t1 // TILE])
    return C, B
