"""Pins of the oracle's backward-pass pieces: the transposed weight layout,
128-token grouping, the GEMM with per-row scales on both operands, and the
data/weight gradients against the float64 product of the dequantized
operands and against exact closed forms."""

import numpy as np
import torch

import oracle
from oracle import quant


def _bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return quant.bf16_bits_to_f32(bits)


def test_weight_transposed_layout():
    rng = np.random.default_rng(1)
    w = _bits(rng.standard_normal((256, 384)) * 0.02)
    q, s, qt, st = oracle.quant_w_128x128_t(w)
    q0, s0 = oracle.quant_w_128x128(w)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    assert qt.shape == (384, 256) and st.shape == (3, 2)
    for k in (0, 127, 128, 383):
        assert np.array_equal(qt[k], q0[:, k])
    assert st[2, 1] == s0[1, 2]


def test_token_groups_brute_force():
    """Each 128-token group of one column: scale = its amax / 448 and codes
    from the argmin encoder, checked column by column."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((256, 40)) * np.exp(rng.standard_normal((1, 40)))
    bits = _bits(x)
    qt, st = oracle.quant_act_128x1_t(bits)
    xf = _f32(bits)
    assert qt.shape == (40, 256) and st.shape == (2, 40)
    tab = oracle.decode_table()
    for n in (0, 17, 39):
        for mb in range(2):
            col = xf[mb * 128:(mb + 1) * 128, n]
            a = np.float32(np.max(np.abs(col)))
            assert st[mb, n] == np.float32(a / np.float32(448.0))
            r = np.float32(np.float32(448.0) / a)
            for j in (0, 5, 127):
                y = float(np.float32(col[j] * r))
                best = min(range(0x7F), key=lambda c: (abs(tab[c] - min(abs(y), 448.0)), c % 2))
                assert qt[n, mb * 128 + j] == best | (0x80 if y < 0 else 0)


def test_rowscaled_reduces_to_block_gemm():
    """Row scales equal to the expanded 128x128 block scales give exactly the
    block-scaled GEMM."""
    rng = np.random.default_rng(3)
    qa, sa = oracle.quant_act_1x128(_bits(rng.standard_normal((20, 256))))
    qb, sb = oracle.quant_w_128x128(_bits(rng.standard_normal((384, 256)) * 0.02))
    sb_rows = np.repeat(sb.T, 128, axis=1)  # [K/128][N]
    C0, B0 = oracle.block_gemm(qa, sa, qb, sb)
    C1, B1 = oracle.block_gemm_rowscaled(qa, sa, qb, sb_rows)
    assert np.array_equal(C0, C1) and np.array_equal(B0, B1)


def test_rowscaled_scalar_brute_force():
    rng = np.random.default_rng(4)
    qa = rng.integers(0, 256, (3, 256)).astype(np.uint8)
    qb = rng.integers(0, 256, (5, 256)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    sa = rng.uniform(0.5, 2, (2, 3)).astype(np.float32)
    sb = rng.uniform(0.5, 2, (2, 5)).astype(np.float32)
    C, _ = oracle.block_gemm_rowscaled(qa, sa, qb, sb)
    tab = oracle.decode_table()
    for m in range(3):
        for n in range(5):
            want = 0.0
            for kb in range(2):
                p = sum(tab[qa[m, k]] * tab[qb[n, k]] for k in range(kb * 128, kb * 128 + 128))
                want += float(sa[kb, m]) * float(sb[kb, n]) * p
            assert abs(C[m, n] - want) <= 1e-12 * max(1.0, abs(want))


def test_gradients_equal_dequantized_products():
    """dX and dW equal the float64 products of the dequantized operands."""
    rng = np.random.default_rng(5)
    M, N, K = 256, 256, 384
    dy = _bits(rng.standard_normal((M, N)) * np.exp(rng.standard_normal((M, 1))))
    w = _bits(rng.standard_normal((N, K)) * 0.02)
    x = _bits(rng.standard_normal((M, K)))
    qdy, sdy, qt, st, C, B = oracle.dgrad(dy, w)
    dyq = oracle.decode(qdy) * np.repeat(sdy.T.astype(np.float64), 128, axis=1)
    wt = oracle.decode(qt) * np.repeat(np.repeat(st.astype(np.float64), 128, 0), 128, 1)
    assert np.all(np.abs(C - dyq @ wt.T) <= 1e-12 * B)
    qdyt, sdyt, qxt, sxt, C2, B2 = oracle.wgrad(dy, x)
    a = oracle.decode(qdyt) * np.repeat(sdyt.T.astype(np.float64), 128, axis=1)
    b = oracle.decode(qxt) * np.repeat(sxt.T.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(C2 - a @ b.T) <= 1e-12 * B2)
    # and the dequantized operands are the inputs within the E4M3 half step
    assert np.allclose(a.T, _f32(dy), rtol=2 ** -4, atol=np.abs(_f32(dy)).max() / 458752)


def test_weight_gradient_closed_form():
    """dY and X on the E4M3 grid with 448 somewhere in every 128-token group
    of every column: all scales are 1 and dW = dY^T X exactly."""
    rng = np.random.default_rng(6)
    tab = oracle.decode_table()
    vals = tab[[c for c in range(256) if c not in (0x7F, 0xFF)]]
    M, N, K = 256, 16, 24
    dy = rng.choice(vals, (M, N))
    x = rng.choice(vals, (M, K))
    dy[::128, :] = 448.0
    x[1::128, :] = -448.0
    qdyt, sdyt, qxt, sxt, C, _ = oracle.wgrad(_bits(dy), _bits(x))
    assert np.all(sdyt == 1.0) and np.all(sxt == 1.0)
    assert np.array_equal(C, dy.T @ x)


def test_zero_token_padding_changes_nothing():
    """Padding a ragged token count with zero rows to a multiple of 128 gives
    the same weight gradient (zeros raise no maximum and add nothing) as
    long as the real tokens fill the first groups; here the last group is
    part real, part padding."""
    rng = np.random.default_rng(7)
    mg, N, K = 200, 16, 24
    dy = rng.standard_normal((mg, N))
    x = rng.standard_normal((mg, K))
    dyp = np.zeros((256, N))
    xp = np.zeros((256, K))
    dyp[:mg] = dy
    xp[:mg] = x
    _, sa, _, sb, C, _ = oracle.wgrad(_bits(dyp), _bits(xp))
    # group 1 holds tokens 128..199 and zeros: its maxima are those of the real tokens
    xf = _f32(_bits(dyp))
    assert np.array_equal(sa[1], np.divide(np.max(np.abs(xf[128:mg]), axis=0).astype(np.float32),
                                           np.float32(448.0), dtype=np.float32))
    # and the gradient equals the sum over the two groups computed from the real tokens only
    a = oracle.decode(oracle.quant_act_128x1_t(_bits(dyp))[0]).T * np.repeat(sa, 128, axis=0)
    b = oracle.decode(oracle.quant_act_128x1_t(_bits(xp))[0]).T * np.repeat(sb, 128, axis=0)
    assert np.allclose(C, a[:mg].T @ b[:mg], rtol=1e-12, atol=0)


def test_kgrouped_equals_per_expert_and_zero_for_empty():
    """The one-call MoE weight gradient is the row-scaled GEMM of each
    expert's token columns (checked against slices computed directly from
    the dequantized operands), and zero for an expert without tokens."""
    rng = np.random.default_rng(8)
    sizes = [256, 0, 128, 384]
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    T, M, N = int(offsets[-1]), 24, 40
    dy = _bits(rng.standard_normal((T, M)))
    x = _bits(rng.standard_normal((T, N)))
    qa, sa = oracle.quant_act_128x1_t(dy)
    qb, sb = oracle.quant_act_128x1_t(x)
    C, B = oracle.kgrouped_gemm_rowscaled(qa, sa, qb, sb, offsets)
    a = oracle.decode(qa) * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    b = oracle.decode(qb) * np.repeat(sb.T.astype(np.float64), 128, axis=1)
    for g in range(4):
        t0, t1 = offsets[g], offsets[g + 1]
        want = a[:, t0:t1] @ b[:, t0:t1].T
        assert np.all(np.abs(C[g] - want) <= 1e-12 * np.maximum(B[g], 1e-300))
    assert not C[1].any() and not B[1].any()
