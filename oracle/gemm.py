"""Block-scaled FP8 GEMM of the oracle, in float64 (test infrastructure only).

What the pages fix
------------------
* "Advantages of using FP8 for GEMM operations in DeepSeek-V3", items 1 and 8:
  the GEMMs run on FP8 operands, for dense and for MoE layers.
* Same page, item 5, and "How the unified E4M3 format adds to DeepSeek-V3's
  efficiency", section "Enhanced numerical stability": partial results are
  promoted into FP32 registers at fixed intervals of the accumulation.

Reading taken: the promotion interval is the 128-wide K group, the same
interval at which the activation-tile and weight-block scales change, so the
operation computed is

    C[m, n] = sum_kb  S_A[kb, m] * S_W[n // 128, kb] * P[m, n, kb]
    P[m, n, kb] = sum_{k in group kb} dec(QA[m, k]) * dec(QW[n, k])

with C = A . W^T (A is [M][K], W is [N][K]).  This is a plain definition, so
it is evaluated directly.  ``P`` is exact in float64: every E4M3 value is a
multiple of 2^-9 below 2^9, so each product is a multiple of 2^-18 below 2^18
and any partial sum of at most 128 of them needs at most 43 significant bits.
The library matmul used for ``P`` therefore returns the exact value whatever
its internal order.  The scaled sum over groups then carries only float64
rounding (relative 2^-52 per term).

Alongside C the oracle returns the tolerance basis
``B[m, n] = sum_kb S_A S_W sum_k |dec(QA) dec(QW)|``; a GPU element is correct
when ``|C_gpu - C| <= 2e-3 * B``.
"""

import numpy as np

from .e4m3 import decode_table
from .quant import TILE, quant_act_1x128, quant_rows_1x128

_DEC = decode_table()


def _col_scale(sw_col, N):
    """Per-column weight scale of one K group: block nb covers 128 columns."""
    return np.repeat(np.asarray(sw_col, dtype=np.float64), TILE)[:N]


def block_gemm(qa, sa, qw, sw):
    """C and its tolerance basis for one dense block-scaled GEMM.

    qa: uint8 [M][K]; sa: float32 [KB][M]; qw: uint8 [N][K];
    sw: float32 [NB][KB].  K must be a multiple of 128.
    Returns ``(C, B)``, both float64 [M][N].
    """
    qa = np.asarray(qa, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and K % TILE == 0
    KB = K // TILE
    C = np.zeros((M, N), dtype=np.float64)
    B = np.zeros((M, N), dtype=np.float64)
    for kb in range(KB):
        k0 = kb * TILE
        a = _DEC[qa[:, k0:k0 + TILE]]
        w = _DEC[qw[:, k0:k0 + TILE]]
        p = a @ w.T
        pabs = np.abs(a) @ np.abs(w).T
        scale = (np.asarray(sa[kb], dtype=np.float64)[:, None]
                 * _col_scale(np.asarray(sw)[:, kb], N)[None, :])
        C += scale * p
        B += scale * pabs
    return C, B


def block_grouped_gemm(qa, sa, qw, sw, offsets, rows=None):
    """Grouped (MoE) block-scaled GEMM.

    Rows ``offsets[g] .. offsets[g+1]-1`` of A multiply expert ``g``'s weight.
    qa: uint8 [M_total][K]; sa: float32 [KB][M_total];
    qw: uint8 [G][N][K]; sw: float32 [G][NB][KB]; offsets: int [G+1].
    ``rows`` optionally selects the rows to compute (default: all).
    Returns ``(C, B)`` float64 [len(rows)][N].
    """
    offsets = np.asarray(offsets, dtype=np.int64)
    G = len(offsets) - 1
    M_total = int(offsets[-1])
    rows = np.arange(M_total) if rows is None else np.asarray(rows, dtype=np.int64)
    N = qw.shape[1]
    C = np.zeros((len(rows), N), dtype=np.float64)
    B = np.zeros((len(rows), N), dtype=np.float64)
    group_of = np.searchsorted(offsets, rows, side="right") - 1
    for g in range(G):
        sel = np.nonzero(group_of == g)[0]
        if sel.size == 0:
            continue
        r = rows[sel]
        c, b = block_gemm(qa[r], np.asarray(sa)[:, r], qw[g], sw[g])
        C[sel] = c
        B[sel] = b
    return C, B


def fused_act_gemm(x_bits, qw, sw):
    """Quantize bf16 activations per 1x128 tile, then the block GEMM.

    Returns ``(qa, sa, C, B)``.
    """
    qa, sa = quant_act_1x128(x_bits)
    C, B = block_gemm(qa, sa, qw, sw)
    return qa, sa, C, B


def block_gemm_e4m3_out(qa, sa, qw, sw):
    """The block GEMM with its output quantized for the next FP8 GEMM.

    C is computed as ``block_gemm``; its float32 rounding RN32(C) is then
    quantized per 1x128 tile along N (``quant_rows_1x128``), the online
    activation rule applied where the FP32 output leaves the GEMM.  A GPU
    quantizes its own FP32 accumulator, which lies within the GEMM tolerance
    of C rather than equal to RN32(C), so its codes are compared with these
    exactly only where C is exact in float32, and by value bounds elsewhere.
    Returns ``(C, B, qc, sc)``; ``sc`` float32 [N/128][M].
    """
    C, B = block_gemm(qa, sa, qw, sw)
    qc, sc = quant_rows_1x128(C.astype(np.float32))
    return C, B, qc, sc
