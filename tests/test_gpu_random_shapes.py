"""Seeded random shapes through the GEMM entry points against the oracle.

Each case draws M, N and K (a multiple of 128) from a fixed generator, so
the launch takes whichever kernel and tile shape it picks for that shape:
the few-row kernels (M <= 64), the 64x128, 128x256 and 256x256 tiles and
their ragged edges.  Every output is checked against the float64 oracle on
the same quantized inputs; activation scales produced inside a call are
compared bit for bit.
"""

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


def _shapes(seed, n, m_max, n_max, k_max):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, m_max + 1)), int(rng.integers(1, n_max + 1)),
             128 * int(rng.integers(1, k_max // 128 + 1))) for _ in range(n)]


# plus two larger ragged shapes that take 256x256 tiles (one round; and four
# rounds with a last partial round of more than half the compute units)
DENSE = _shapes(7001, 12, 1500, 3000, 512) + [(2300, 7100, 256), (4200, 18000, 128)]
BF16_A = _shapes(7002, 8, 200, 1200, 768)
ROWSCALED = _shapes(7003, 6, 1200, 1200, 512)


def _operands(M, N, K, case):
    a = synth.act(M, K, case=case, tensor=0)
    w = synth.weight(N, K, case=case, tensor=1)
    return synth.bf16_bits(a), synth.bf16_bits(w)


@pytest.mark.parametrize("i", range(len(DENSE)))
def test_random_dense(fp8bs, i):
    M, N, K = DENSE[i]
    out = torch.bfloat16 if i % 2 else torch.float32
    ab, wb = _operands(M, N, K, case=900 + i)
    qa, sa = oracle.quant_act_1x128(ab)
    qw, sw = oracle.quant_w_128x128(wb)
    c = fp8bs.fp8_block_gemm(gu.u8(qa), gu.f32(sa), gu.u8(qw), gu.f32(sw), out_dtype=out)
    torch.cuda.synchronize()
    C, B = oracle.block_gemm(qa, sa, qw, sw)
    gu.check_gemm(c, C, B)


@pytest.mark.parametrize("i", range(len(BF16_A)))
def test_random_bf16_activation(fp8bs, i):
    """bf16 A quantized inside the call (the few-row kernels quantize it in
    the GEMM kernel at M <= 16)."""
    M, N, K = BF16_A[i]
    ab, wb = _operands(M, N, K, case=920 + i)
    qw, sw = oracle.quant_w_128x128(wb)
    sa_out = torch.empty(K // 128, M, dtype=torch.float32, device="cuda")
    c = fp8bs.fp8_block_gemm(gu.bf16_from_bits(ab), sa_out, gu.u8(qw), gu.f32(sw),
                             out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _, sa, C, B = oracle.fused_act_gemm(ab, qw, sw)
    gu.assert_same_bits(gu.host(sa_out), sa, "in-call activation scales")
    gu.check_gemm(c, C, B)


@pytest.mark.parametrize("i", range(8))
def test_random_grouped(fp8bs, i):
    rng = np.random.default_rng(7100 + i)
    G = int(rng.integers(1, 13))
    # group sizes with empty groups and sizes around the tile heights
    sizes = [int(rng.choice([0, 1, 127, 128, 129, 255, 256, 257, int(rng.integers(1, 600))]))
             for _ in range(G)]
    N = int(rng.integers(1, 1100))
    K = 128 * int(rng.integers(1, 5))
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(offsets[-1])
    if M == 0:
        pytest.skip("all groups drawn empty")
    case = 940 + i
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(synth.act(M, K, case=case, tensor=0)))
    qws, sws = [], []
    for g in range(G):
        q, s = oracle.quant_w_128x128(synth.bf16_bits(synth.weight(N, K, case=case, tensor=10 + g)))
        qws.append(q)
        sws.append(s)
    qw, sw = np.stack(qws), np.stack(sws)
    out = torch.bfloat16 if i % 2 else torch.float32
    c = fp8bs.fp8_block_grouped_gemm(gu.u8(qa), gu.f32(sa), gu.u8(qw), gu.f32(sw),
                                     torch.from_numpy(offsets).cuda(), out_dtype=out)
    torch.cuda.synchronize()
    C, B = oracle.block_grouped_gemm(qa, sa, qw, sw, offsets)
    gu.check_gemm(c, C, B)


@pytest.mark.parametrize("i", range(len(ROWSCALED)))
def test_random_rowscaled(fp8bs, i):
    """One scale per row and 128-K group on both operands (the weight
    gradient's form)."""
    M, N, K = ROWSCALED[i]
    case = 960 + i
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(synth.act(M, K, case=case, tensor=0)))
    qb, sb = oracle.quant_act_1x128(synth.bf16_bits(synth.act(N, K, case=case, tensor=1)))
    out = torch.bfloat16 if i % 2 else torch.float32
    c = fp8bs.fp8_block_gemm_rowscaled(gu.u8(qa), gu.f32(sa), gu.u8(qb), gu.f32(sb),
                                       out_dtype=out)
    torch.cuda.synchronize()
    C, B = oracle.block_gemm_rowscaled(qa, sa, qb, sb)
    gu.check_gemm(c, C, B)
