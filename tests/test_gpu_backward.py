"""GPU parity of the backward-pass pieces against the oracle: the transposed
weight quantizer and the 128-token quantizer (bit-exact), the GEMM with
per-row scales on both operands, and the data and weight gradients end to
end (GPU quantizers, then GPU GEMMs, against the oracle on the same bf16
inputs)."""

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_05_amd import synth
from tests import _gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    from fp8_block_scaled_05_amd import fp8bs as mod
    return mod


@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (384, 1024)])
def test_weight_quantizer_transposed_bit_exact(fp8bs, N, K):
    w = synth.weight(N, K, case=800 + N, tensor=1)
    q, s, qt, st = fp8bs.fp8_quant_w_128x128_t(w.cuda())
    torch.cuda.synchronize()
    q_o, s_o, qt_o, st_o = oracle.quant_w_128x128_t(synth.bf16_bits(w))
    gu.assert_same_bits(gu.host(q), q_o, "codes")
    gu.assert_same_bits(gu.host(s), s_o, "scales")
    gu.assert_same_bits(gu.host(qt), qt_o, "transposed codes")
    gu.assert_same_bits(gu.host(st), st_o, "transposed scales")


@pytest.mark.parametrize("M,N", [(128, 128), (256, 384), (640, 256)])
def test_token_group_quantizer_bit_exact(fp8bs, M, N):
    x = synth.act(M, N, case=810 + M, tensor=0)
    qt, st = fp8bs.fp8_quant_act_128x1_t(x.cuda())
    torch.cuda.synchronize()
    qt_o, st_o = oracle.quant_act_128x1_t(synth.bf16_bits(x))
    gu.assert_same_bits(gu.host(qt), qt_o, "codes")
    gu.assert_same_bits(gu.host(st), st_o, "scales")


def test_token_group_quantizer_strided(fp8bs):
    M, N = 256, 256
    X = synth.act(M, N + 64, case=815, tensor=0).cuda()
    QT = torch.full((N, M + 32), 0x33, dtype=torch.uint8, device="cuda")
    ST = torch.full((M // 128, N + 8), -1.0, dtype=torch.float32, device="cuda")
    fp8bs.fp8_quant_act_128x1_t(X[:, :N], qt=QT[:, :M], st=ST)
    torch.cuda.synchronize()
    qt_o, st_o = oracle.quant_act_128x1_t(synth.bf16_bits(X[:, :N]))
    gu.assert_same_bits(gu.host(QT[:, :M]), qt_o, "codes")
    gu.assert_same_bits(gu.host(ST[:, :N]), st_o, "scales")
    assert torch.all(QT[:, M:] == 0x33) and torch.all(ST[:, N:] == -1.0)


@pytest.mark.parametrize("M,N,K,out", [
    (300, 384, 512, torch.float32),   # 64x128 tiles (too few 256x256 ones), ragged M
    (1000, 4000, 256, torch.bfloat16),  # 128x256 tiles, ragged M and N
    (257, 200, 256, torch.bfloat16),  # ragged N
    (48, 256, 384, torch.float32),    # few-row tile
    (20, 72, 256, torch.float32),     # 32x32 tile, ragged
])
def test_rowscaled_gemm(fp8bs, M, N, K, out):
    a = synth.act(M, K, case=820 + M, tensor=0)
    b = synth.act(N, K, case=820 + M, tensor=1)
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(a))
    qb, sb = oracle.quant_act_1x128(synth.bf16_bits(b))
    c = fp8bs.fp8_block_gemm_rowscaled(gu.u8(qa), gu.f32(sa), gu.u8(qb), gu.f32(sb),
                                       out_dtype=out)
    torch.cuda.synchronize()
    C, B = oracle.block_gemm_rowscaled(qa, sa, qb, sb)
    gu.check_gemm(c, C, B)


def test_rowscaled_gemm_strided(fp8bs):
    """Operands and scales inside wider buffers (lda, ldb > K; ldsa > M,
    ldsb > N; ldc > N): the padding is neither read into the result nor
    written."""
    M, N, K = 130, 200, 384
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(synth.act(M, K, case=825, tensor=0)))
    qb, sb = oracle.quant_act_1x128(synth.bf16_bits(synth.act(N, K, case=825, tensor=1)))
    A = torch.full((M, K + 32), 0x7E, dtype=torch.uint8, device="cuda")
    B = torch.full((N, K + 48), 0x7E, dtype=torch.uint8, device="cuda")
    SA = torch.full((K // 128, M + 6), 1e30, dtype=torch.float32, device="cuda")
    SB = torch.full((K // 128, N + 10), 1e30, dtype=torch.float32, device="cuda")
    A[:, :K] = gu.u8(qa)
    B[:, :K] = gu.u8(qb)
    SA[:, :M] = gu.f32(sa)
    SB[:, :N] = gu.f32(sb)
    C = torch.full((M, N + 16), -3.0, dtype=torch.float32, device="cuda")
    fp8bs.fp8_block_gemm_rowscaled(A[:, :K], SA, B[:, :K], SB, out=C[:, :N])
    torch.cuda.synchronize()
    Cr, Br = oracle.block_gemm_rowscaled(qa, sa, qb, sb)
    gu.check_gemm(C[:, :N], Cr, Br)
    assert torch.all(C[:, N:] == -3.0)


def test_weight_quantizer_transposed_strided(fp8bs):
    N, K = 256, 384
    w = synth.weight(N, K + 64, case=805, tensor=1).cuda()
    Q = torch.full((N, K + 16), 0x11, dtype=torch.uint8, device="cuda")
    QT = torch.full((K, N + 32), 0x22, dtype=torch.uint8, device="cuda")
    s = torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")
    st = torch.empty(K // 128, N // 128, dtype=torch.float32, device="cuda")
    fp8bs.fp8_quant_w_128x128_t(w[:, :K], q=Q[:, :K], s=s, qt=QT[:, :N], st=st)
    torch.cuda.synchronize()
    q_o, s_o, qt_o, st_o = oracle.quant_w_128x128_t(synth.bf16_bits(w[:, :K]))
    gu.assert_same_bits(gu.host(Q[:, :K]), q_o, "codes")
    gu.assert_same_bits(gu.host(QT[:, :N]), qt_o, "transposed codes")
    gu.assert_same_bits(gu.host(st), st_o, "transposed scales")
    assert torch.all(Q[:, K:] == 0x11) and torch.all(QT[:, N:] == 0x22)


def test_rowscaled_gemm_adversarial_scales(fp8bs):
    """Per-row, per-group scales spanning 2^+-20 on both operands: a kernel
    that applied either scale outside the per-group promotion, or to the
    wrong row or column, would fail the tolerance."""
    M, N, K = 130, 260, 1024
    rng = np.random.default_rng(21)
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(synth.act(M, K, case=830, tensor=0)))
    qb, sb = oracle.quant_act_1x128(synth.bf16_bits(synth.act(N, K, case=830, tensor=1)))
    sa = (sa * np.float32(2.0) ** rng.integers(-20, 21, sa.shape)).astype(np.float32)
    sb = (sb * np.float32(2.0) ** rng.integers(-20, 21, sb.shape)).astype(np.float32)
    c = fp8bs.fp8_block_gemm_rowscaled(gu.u8(qa), gu.f32(sa), gu.u8(qb), gu.f32(sb))
    torch.cuda.synchronize()
    C, B = oracle.block_gemm_rowscaled(qa, sa, qb, sb)
    gu.check_gemm(c, C, B)


def test_rowscaled_gemm_last_round_split(fp8bs):
    """272 tiles (> 256 compute units, not whole rounds): the last partial
    round runs as half-height tiles with row-scaled B as well."""
    M, N, K = 4352, 4096, 128
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(synth.act(M, K, case=835, tensor=0)))
    qb, sb = oracle.quant_act_1x128(synth.bf16_bits(synth.act(N, K, case=835, tensor=1)))
    c = fp8bs.fp8_block_gemm_rowscaled(gu.u8(qa), gu.f32(sa), gu.u8(qb), gu.f32(sb))
    torch.cuda.synchronize()
    C, B = oracle.block_gemm_rowscaled(qa, sa, qb, sb)
    gu.check_gemm(c, C, B)


def test_data_gradient_end_to_end(fp8bs):
    """dX = dY . W: dY quantized per 1x128 along N, W per 128x128 block read
    transposed; every output against the oracle."""
    M, N, K = 300, 384, 256
    dy = synth.act(M, N, case=840, tensor=0)
    w = synth.weight(N, K, case=840, tensor=1)
    qdy, sdy = fp8bs.fp8_quant_act_1x128(dy.cuda())
    _, _, qt, st = fp8bs.fp8_quant_w_128x128_t(w.cuda())
    dx = fp8bs.fp8_block_gemm(qdy, sdy, qt, st, out_dtype=torch.float32)
    torch.cuda.synchronize()
    qdy_o, sdy_o, qt_o, st_o, C, B = oracle.dgrad(synth.bf16_bits(dy), synth.bf16_bits(w))
    gu.assert_same_bits(gu.host(qdy), qdy_o, "dY codes")
    gu.assert_same_bits(gu.host(qt), qt_o, "W^T codes")
    gu.check_gemm(dx, C, B)


def test_weight_gradient_end_to_end(fp8bs):
    """dW = dY^T . X: both quantized in 128-token groups; every output
    against the oracle."""
    M, N, K = 384, 256, 384
    dy = synth.act(M, N, case=850, tensor=0)
    x = synth.act(M, K, case=850, tensor=1)
    qdyt, sdyt = fp8bs.fp8_quant_act_128x1_t(dy.cuda())
    qxt, sxt = fp8bs.fp8_quant_act_128x1_t(x.cuda())
    dw = fp8bs.fp8_block_gemm_rowscaled(qdyt, sdyt, qxt, sxt)
    torch.cuda.synchronize()
    qdyt_o, _, qxt_o, _, C, B = oracle.wgrad(synth.bf16_bits(dy), synth.bf16_bits(x))
    gu.assert_same_bits(gu.host(qdyt), qdyt_o, "dY^T codes")
    gu.assert_same_bits(gu.host(qxt), qxt_o, "X^T codes")
    gu.check_gemm(dw, C, B)


def test_full_size_gradients_sampled(fp8bs):
    """Backward of the dense layer at full size (tokens M=4096, N=18432,
    K=7168): dX [4096][7168] (contraction 18432, bf16) and dW [18432][7168]
    (contraction 4096, fp32).  Sampled rows x sampled 128-column blocks
    against the oracle, which needs only those columns of W and X."""
    M, N, K = 4096, 18432, 7168
    dy = synth.act(M, N, case=synth.DENSE.case_id, tensor=20, device="cuda")
    w = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    x = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    qdy, sdy = fp8bs.fp8_quant_act_1x128(dy)
    _, _, qt, st = fp8bs.fp8_quant_w_128x128_t(w)
    dx = fp8bs.fp8_block_gemm(qdy, sdy, qt, st, out_dtype=torch.bfloat16)
    qdyt, sdyt = fp8bs.fp8_quant_act_128x1_t(dy)
    qxt, sxt = fp8bs.fp8_quant_act_128x1_t(x)
    dw = fp8bs.fp8_block_gemm_rowscaled(qdyt, sdyt, qxt, sxt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    kbs = sorted(set([0, K // 128 - 1] + rng.choice(K // 128, 2, replace=False).tolist()))
    dy_bits = synth.bf16_bits(dy)
    w_bits = synth.bf16_bits(w)
    x_bits = synth.bf16_bits(x)
    dx_h, dw_h = gu.host_f64(dx), gu.host_f64(dw)
    qt_h, qxt_h = gu.host(qt), gu.host(qxt)
    # data gradient: sampled rows of dY, all N, output column blocks kb
    rows = np.array(sorted(set([0, M - 1] + rng.choice(M, 4, replace=False).tolist())))
    qd, sd = oracle.quant_act_1x128(dy_bits[rows])
    gu.assert_same_bits(gu.host(qdy)[rows], qd, "sampled dY codes")
    # weight gradient: sampled rows n of dW (columns of dY), all tokens
    ns = np.array(sorted(set([0, N - 1] + rng.choice(N, 4, replace=False).tolist())))
    qa_o, sa_o = oracle.quant_act_128x1_t(dy_bits[:, ns])
    gu.assert_same_bits(gu.host(qdyt)[ns], qa_o, "sampled dY^T codes")
    for kb in kbs:
        cols = slice(kb * 128, (kb + 1) * 128)
        _, _, qt_o, st_o = oracle.quant_w_128x128_t(w_bits[:, cols])
        gu.assert_same_bits(qt_h[cols], qt_o, f"W^T codes, block {kb}")
        C, B = oracle.block_gemm(qd, sd, qt_o, st_o)
        gu.check_gemm(dx_h[rows][:, cols], C, B, bf16=True)
        qb_o, sb_o = oracle.quant_act_128x1_t(x_bits[:, cols])
        gu.assert_same_bits(qxt_h[cols], qb_o, f"X^T codes, block {kb}")
        C2, B2 = oracle.block_gemm_rowscaled(qa_o, sa_o, qb_o, sb_o)
        gu.check_gemm(dw_h[ns][:, cols], C2, B2)


def test_moe_data_gradient_grouped(fp8bs):
    """MoE data gradient dX_g = dY_g . W_g with the grouped GEMM: each
    expert's weight quantized with its transposed copy; the stacked
    [G][K][N] codes and [G][K/128][N/128] scales are the grouped call's
    expert layout.  Every output against the oracle, expert by expert."""
    sizes = [70, 0, 300, 129, 5]
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    G, M, N, K = len(sizes), int(offsets[-1]), 256, 384
    dy = synth.act(M, N, case=860, tensor=0)
    ws = [synth.weight(N, K, case=860, tensor=10 + g) for g in range(G)]
    qt = torch.empty(G, K, N, dtype=torch.uint8, device="cuda")
    st = torch.empty(G, K // 128, N // 128, dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8bs.fp8_quant_w_128x128_t(ws[g].cuda(), qt=qt[g], st=st[g])
    qdy, sdy = fp8bs.fp8_quant_act_1x128(dy.cuda())
    dx = fp8bs.fp8_block_grouped_gemm(qdy, sdy, qt, st, torch.from_numpy(offsets).cuda(),
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    dx_h = gu.host_f64(dx)
    for g, (r0, r1) in enumerate(zip(offsets[:-1], offsets[1:])):
        if r1 == r0:
            continue
        _, _, qt_o, st_o, C, B = oracle.dgrad(synth.bf16_bits(dy[r0:r1]), synth.bf16_bits(ws[g]))
        gu.assert_same_bits(gu.host(qt[g]), qt_o, f"expert {g} W^T codes")
        gu.check_gemm(dx_h[r0:r1], C, B)


def test_moe_weight_gradient_per_expert(fp8bs):
    """MoE weight gradient dW_g = dY_g^T . X_g over each expert's tokens,
    padded with zero rows to a multiple of 128 (zeros change neither the
    group maxima nor the sums): the padded oracle equals the unpadded
    definition, and the GPU matches it."""
    sizes = [70, 300, 129]
    N, K = 128, 256
    rng_case = 870
    for g, mg in enumerate(sizes):
        dy = synth.act(mg, N, case=rng_case, tensor=g)
        x = synth.act(mg, K, case=rng_case, tensor=100 + g)
        mp = (mg + 127) // 128 * 128
        dyp = torch.zeros(mp, N, dtype=torch.bfloat16)
        xp = torch.zeros(mp, K, dtype=torch.bfloat16)
        dyp[:mg] = dy
        xp[:mg] = x
        qa, sa = fp8bs.fp8_quant_act_128x1_t(dyp.cuda())
        qb, sb = fp8bs.fp8_quant_act_128x1_t(xp.cuda())
        dw = fp8bs.fp8_block_gemm_rowscaled(qa, sa, qb, sb)
        torch.cuda.synchronize()
        qa_o, sa_o, qb_o, sb_o, C, B = oracle.wgrad(synth.bf16_bits(dyp), synth.bf16_bits(xp))
        gu.assert_same_bits(gu.host(qa), qa_o, f"expert {g} dY^T codes")
        gu.assert_same_bits(gu.host(qb), qb_o, f"expert {g} X^T codes")
        gu.check_gemm(dw, C, B)


def _token_groups(sizes, M, N, case):
    """Per-expert dY [mg][M] and X [mg][N], zero-padded to multiples of 128 and
    concatenated; returns the padded bf16 tensors and the padded offsets."""
    padded = [(mg + 127) // 128 * 128 for mg in sizes]
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    T = int(offsets[-1])
    dy = torch.zeros(T, M, dtype=torch.bfloat16)
    x = torch.zeros(T, N, dtype=torch.bfloat16)
    for g, mg in enumerate(sizes):
        if mg:
            dy[offsets[g]:offsets[g] + mg] = synth.act(mg, M, case=case, tensor=g)
            x[offsets[g]:offsets[g] + mg] = synth.act(mg, N, case=case, tensor=100 + g)
    return dy, x, offsets


@pytest.mark.parametrize("sizes,M,N,out,gpu_quant", [
    ([200, 0, 70, 300], 300, 200, torch.float32, False),  # ragged rows/cols, an empty expert
    ([128] * 20, 1024, 1024, torch.float32, True),        # 320 tiles: last round as half tiles
    ([129, 1, 256], 256, 384, torch.bfloat16, True),
])
def test_kgrouped_weight_gradient(fp8bs, sizes, M, N, out, gpu_quant):
    """One launch over all experts against the oracle, expert by expert; the
    operands come from the GPU quantizers (checked bit for bit) or, for
    feature sizes the transposed quantizer does not take, from the oracle."""
    dy, x, offsets = _token_groups(sizes, M, N, case=880 + len(sizes))
    qa_o, sa_o = oracle.quant_act_128x1_t(synth.bf16_bits(dy))
    qb_o, sb_o = oracle.quant_act_128x1_t(synth.bf16_bits(x))
    if gpu_quant:
        qa, sa = fp8bs.fp8_quant_act_128x1_t(dy.cuda())
        qb, sb = fp8bs.fp8_quant_act_128x1_t(x.cuda())
        torch.cuda.synchronize()
        gu.assert_same_bits(gu.host(qa), qa_o, "dY^T codes")
        gu.assert_same_bits(gu.host(qb), qb_o, "X^T codes")
    else:
        qa, sa, qb, sb = gu.u8(qa_o), gu.f32(sa_o), gu.u8(qb_o), gu.f32(sb_o)
    G = len(sizes)
    dw = torch.full((G, M, N), 5.0, dtype=out, device="cuda")
    fp8bs.fp8_block_kgrouped_gemm_rowscaled(qa, sa, qb, sb, torch.from_numpy(offsets).cuda(),
                                            out=dw)
    torch.cuda.synchronize()
    C, B = oracle.kgrouped_gemm_rowscaled(qa_o, sa_o, qb_o, sb_o, offsets)
    dwh = gu.host_f64(dw)
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(dwh[g] == 0.0), f"expert {g} without tokens must be zero"
        else:
            gu.check_gemm(dwh[g], C[g], B[g], bf16=out == torch.bfloat16)


def test_kgrouped_offsets_outside_the_contract_stay_in_bounds(fp8bs):
    """Expert ranges out of order and past the end are clamped on the device:
    expert 0 over tokens [0, 256), expert 1 empty (its end 128 is raised to
    its start 256), expert 2 over [128, T) (its end T + 128 is lowered to T).
    Each expert has its own output, so every result stays defined."""
    M, N = 256, 128
    dy, x, _ = _token_groups([384], M, N, case=890)
    T = dy.shape[0]
    qa_o, sa_o = oracle.quant_act_128x1_t(synth.bf16_bits(dy))
    qb_o, sb_o = oracle.quant_act_128x1_t(synth.bf16_bits(x))
    offsets = np.array([0, 256, 128, T + 128], dtype=np.int32)
    dw = torch.full((3, M, N), 5.0, dtype=torch.float32, device="cuda")
    fp8bs.fp8_block_kgrouped_gemm_rowscaled(gu.u8(qa_o), gu.f32(sa_o), gu.u8(qb_o), gu.f32(sb_o),
                                            torch.from_numpy(offsets).cuda(), out=dw)
    torch.cuda.synchronize()
    dwh = gu.host_f64(dw)
    C0, B0 = oracle.block_gemm_rowscaled(qa_o[:, :256], sa_o[:2], qb_o[:, :256], sb_o[:2])
    gu.check_gemm(dwh[0], C0, B0)
    assert np.all(dwh[1] == 0.0)
    C2, B2 = oracle.block_gemm_rowscaled(qa_o[:, 128:T], sa_o[1:], qb_o[:, 128:T], sb_o[1:])
    gu.check_gemm(dwh[2], C2, B2)
