"""Pins of the oracle's block-scaled GEMM: pure-Python brute force, a second
evaluation with scales folded into the operands, the identity-scale special
case (a plain matmul), one-hot indexing, the promotion adversary, the grouped
variant and planted mistakes."""

import numpy as np
import pytest
import torch

import oracle
from oracle import gemm as ogemm
from oracle import quant as oquant


def _bf16_bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _operands(M, N, K, seed=0, outliers=True):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K))
    if outliers:
        idx = rng.choice(M * K, max(1, M * K // 1000), replace=False)
        a.ravel()[idx] *= 50.0
    w = rng.standard_normal((N, K)) * 0.02
    qa, sa = oracle.quant_act_1x128(_bf16_bits(a))
    qw, sw = oracle.quant_w_128x128(_bf16_bits(w))
    return qa, sa, qw, sw


def _brute(qa, sa, qw, sw):
    """Definition written out with scalar loops (float64)."""
    tab = oracle.decode_table().tolist()
    M, K = qa.shape
    N = qw.shape[0]
    C = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for kb in range(K // 128):
                p = 0.0
                for k in range(kb * 128, kb * 128 + 128):
                    p += tab[qa[m, k]] * tab[qw[n, k]]
                acc += float(sa[kb, m]) * float(sw[n // 128, kb]) * p
            C[m][n] = acc
    return np.array(C)


def test_matches_scalar_brute_force():
    qa, sa, qw, sw = _operands(3, 136, 256, seed=1)
    C, B = oracle.block_gemm(qa, sa, qw, sw)
    ref = _brute(qa, sa, qw, sw)
    assert np.allclose(C, ref, rtol=1e-13, atol=0)


def test_matches_folded_scale_matmul():
    """Scales folded into dequantized operands, one float64 matmul over K."""
    qa, sa, qw, sw = _operands(64, 384, 512, seed=2)
    a = oracle.decode(qa) * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    wsc = np.repeat(np.repeat(sw.astype(np.float64), 128, axis=0), 128, axis=1)[:384]
    w = oracle.decode(qw) * wsc
    C, B = oracle.block_gemm(qa, sa, qw, sw)
    # cancellation makes a relative bound on C meaningless; bound by B
    assert np.all(np.abs(C - a @ w.T) <= 1e-12 * B)
    assert np.allclose(B, np.abs(a) @ np.abs(w).T, rtol=1e-12)


def test_identity_scale_case_is_plain_matmul():
    """E4M3-representable inputs whose every tile/block maximum is exactly 448
    quantize with s = r = 1 and no rounding, so the GEMM is a plain matmul."""
    rng = np.random.default_rng(3)
    tab = oracle.decode_table()
    finite = tab[[c for c in range(256) if c not in (0x7F, 0xFF)]]
    M, N, K = 16, 256, 384
    a = rng.choice(finite, (M, K))
    w = rng.choice(finite, (N, K))
    a[:, ::128] = 448.0
    w[::128, :] = -448.0
    qa, sa = oracle.quant_act_1x128(_bf16_bits(a))
    qw, sw = oracle.quant_w_128x128(_bf16_bits(w))
    assert np.all(sa == 1.0) and np.all(sw == 1.0)
    C, _ = oracle.block_gemm(qa, sa, qw, sw)
    assert np.array_equal(C, a @ w.T)


def test_one_hot_pins_indexing():
    qa, sa, qw, sw = _operands(8, 384, 512, seed=4)
    m0, k0 = 5, 300
    kb0 = k0 // 128
    qa1 = np.zeros_like(qa)
    qa1[m0, k0] = 0x45  # 3.25
    C, _ = oracle.block_gemm(qa1, sa, qw, sw)
    tab = oracle.decode_table()
    want = np.zeros_like(C)
    want[m0] = (float(sa[kb0, m0]) * np.repeat(sw[:, kb0].astype(np.float64), 128)[:384]
                * 3.25 * tab[qw[:, k0]])
    assert np.array_equal(C, want)


def _promotion_adversary(M=4, N=256, K=1024, seed=5):
    qa, sa, qw, sw = _operands(M, N, K, seed=seed)
    rng = np.random.default_rng(seed)
    sa = (sa * np.float32(2.0) ** rng.integers(-20, 21, sa.shape)).astype(np.float32)
    sw = (sw * np.float32(2.0) ** rng.integers(-20, 21, sw.shape)).astype(np.float32)
    return qa, sa, qw, sw


def test_promotion_adversary_rejects_late_scaling():
    """With per-group scales spanning 2^+-20 inside one row, applying one
    averaged scale after the full-K sum is far outside the tolerance."""
    qa, sa, qw, sw = _promotion_adversary()
    C, B = oracle.block_gemm(qa, sa, qw, sw)
    tab = oracle.decode_table()
    P = oracle.decode(qa) @ oracle.decode(qw).T
    late = P * np.mean(sa, axis=0)[:, None] * np.repeat(np.mean(sw, axis=1), 128)[None, :]
    assert np.mean(np.abs(late - C) > 2e-3 * B) > 0.5


def _fp32_model(qa, sa, qw, sw):
    """What an FP32-promoting kernel computes: each 128-K partial sum in
    float32, promoted by one float32 multiply-add per group, bf16 output."""
    M, K = qa.shape
    N = qw.shape[0]
    acc = np.zeros((M, N), dtype=np.float32)
    for kb in range(K // 128):
        a = oracle.decode(qa[:, kb * 128:(kb + 1) * 128]).astype(np.float32)
        w = oracle.decode(qw[:, kb * 128:(kb + 1) * 128]).astype(np.float32)
        p = (a @ w.T).astype(np.float32)
        sc = (sa[kb][:, None] * np.repeat(sw[:, kb], 128)[:N][None, :]).astype(np.float32)
        acc = (acc + p * sc).astype(np.float32)
    return torch.from_numpy(acc).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("adversary", [False, True])
def test_fp32_promotion_meets_tolerance(adversary):
    """The 2e-3 * sum|a b| tolerance is met by FP32 promotion with bf16 output
    (so the reading of the bar is attainable), including the adversary."""
    ops = _promotion_adversary() if adversary else _operands(32, 256, 1024, seed=6)
    C, B = oracle.block_gemm(*ops)
    got = _fp32_model(*ops)
    assert np.all(np.abs(got - C) <= 2e-3 * B)


def test_grouped_equals_dense_slices_with_empty_groups():
    rng = np.random.default_rng(7)
    G, N, K = 5, 256, 256
    sizes = np.array([3, 0, 17, 0, 9])
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    M = int(offsets[-1])
    qa, sa = oracle.quant_act_1x128(_bf16_bits(rng.standard_normal((M, K))))
    qws, sws = [], []
    for g in range(G):
        q, s = oracle.quant_w_128x128(_bf16_bits(rng.standard_normal((N, K)) * 0.02))
        qws.append(q)
        sws.append(s)
    qw, sw = np.stack(qws), np.stack(sws)
    C, B = oracle.block_grouped_gemm(qa, sa, qw, sw, offsets)
    for g in range(G):
        r0, r1 = offsets[g], offsets[g + 1]
        if r1 == r0:
            continue
        c, b = oracle.block_gemm(qa[r0:r1], sa[:, r0:r1], qw[g], sw[g])
        assert np.array_equal(C[r0:r1], c) and np.array_equal(B[r0:r1], b)
    rows = np.array([0, 20, 28])
    Cs, _ = oracle.block_grouped_gemm(qa, sa, qw, sw, offsets, rows=rows)
    assert np.array_equal(Cs, C[rows])


def test_fused_is_quant_then_gemm():
    rng = np.random.default_rng(8)
    x = _bf16_bits(rng.standard_normal((16, 256)))
    qw, sw = oracle.quant_w_128x128(_bf16_bits(rng.standard_normal((128, 256)) * 0.02))
    qa, sa, C, B = oracle.fused_act_gemm(x, qw, sw)
    qa2, sa2 = oracle.quant_act_1x128(x)
    assert np.array_equal(qa, qa2) and np.array_equal(sa, sa2)
    assert np.array_equal(C, oracle.block_gemm(qa2, sa2, qw, sw)[0])


def test_planted_mistakes_are_caught(monkeypatch):
    """Plant plausible slips in the oracle (CPU only) and check that a pin
    above fails for each."""
    qa, sa, qw, sw = _operands(8, 384, 512, seed=4)

    def one_hot_ok():
        m0, k0 = 5, 300
        qa1 = np.zeros_like(qa)
        qa1[m0, k0] = 0x45
        C, _ = oracle.block_gemm(qa1, sa, qw, sw)
        kb0 = k0 // 128
        want = np.zeros_like(C)
        want[m0] = (float(sa[kb0, m0]) * np.repeat(sw[:, kb0].astype(np.float64), 128)[:384]
                    * 3.25 * oracle.decode_table()[qw[:, k0]])
        return np.array_equal(C, want)

    assert one_hot_ok()
    # (1) weight scale indexed with the K group as the row: transposed grid
    orig = ogemm._col_scale
    monkeypatch.setattr(ogemm, "_col_scale", lambda col, N: orig(np.roll(col, 1), N))
    assert not one_hot_ok()
    monkeypatch.setattr(ogemm, "_col_scale", orig)
    # (2) dropped activation scale
    real = oracle.block_gemm
    C0 = real(qa, sa, qw, sw)[0]
    C1 = real(qa, np.ones_like(sa), qw, sw)[0]
    assert not np.allclose(C0, C1)
    # (3) quantizer dividing by 127 instead of mapping amax to 448
    monkeypatch.setattr(oquant, "_F448", np.float32(127.0))
    q, s = oracle.quant_act_1x128(np.array([[0x3F80] * 128], dtype=np.uint16))
    assert q[0, 0] != 0x7E


def test_e4m3_out_closed_form():
    """One-hot activation rows (448 at column k0(m), zero elsewhere) and a
    weight on the E4M3 grid whose every 128x128 block and every column of a
    128-row band reach 448: s_A = s_W = 1, C[m, n] = 448 * w[n, k0(m)]
    exactly, and its 1x128 output tiles have amax 448 * 448, so the output
    scale is exactly 448 and the output codes are the weight's own codes."""
    rng = np.random.default_rng(9)
    tab = oracle.decode_table()
    # -0 is left out: the sum C = 0 + 448 * (-0) is +0, whose code differs
    finite = tab[[c for c in range(256) if c not in (0x7F, 0xFF, 0x80)]]
    M, N, K = 8, 384, 256
    w = rng.choice(finite, (N, K))
    w[::128, :] = 448.0
    k0 = rng.integers(0, K, M)
    a = np.zeros((M, K))
    a[np.arange(M), k0] = 448.0
    qa, sa = oracle.quant_act_1x128(_bf16_bits(a))
    qw, sw = oracle.quant_w_128x128(_bf16_bits(w))
    assert np.all(sw == 1.0)
    C, B, qc, sc = oracle.block_gemm_e4m3_out(qa, sa, qw, sw)
    assert np.array_equal(C, 448.0 * w[:, k0].T)
    assert sc.shape == (N // 128, M) and np.all(sc == 448.0)
    assert np.array_equal(qc, qw[:, k0].T)
    # the quantized output decodes back to C within the E4M3 half-ulp bound
    deq = oracle.decode(qc) * np.repeat(sc.T.astype(np.float64), 128, axis=1)
    assert np.array_equal(deq, C)
