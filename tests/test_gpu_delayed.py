"""GPU parity of delayed (history-based) scaling against the oracle: codes,
scales and the clipped/flushed counts bit for bit over multi-step sequences
of drifting activations, and the device history ring against its storage
contract (built here from the oracle's per-step maxima)."""

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


def _expected_ring(past, t, H, mode, KB, M):
    """The device history ring after step t, from the per-step maxima
    ``past`` (steps 0..t): the storage contract of fp8_quant_act_1x128_delayed.
    Per tile, ring [H][KB][M]: step u lives in slot u % H.  Per tensor, ring
    [H + 2]: step u lives in slot u % (H + 2) and slot (t + 1) % (H + 2), the
    slot the next step raises, is clear."""
    if mode == "tile":
        ring = np.zeros((H, KB, M), np.float32)
        for u in range(max(0, t - H + 1), t + 1):
            ring[u % H] = past[u]
    else:
        ring = np.zeros(H + 2, np.float32)
        for u in range(max(0, t - H), t + 1):
            ring[u % (H + 2)] = past[u]
        ring[(t + 1) % (H + 2)] = 0.0
    return ring


@pytest.mark.parametrize("mode,H,M,K,ldh_pad,growth", [
    ("tile", 1, 64, 256, 0, 1.05),
    ("tile", 4, 70, 384, 6, 1.3),
    ("tile", 3, 1, 128, 0, 0.8),
    ("tensor", 1, 64, 256, 0, 1.05),
    ("tensor", 3, 100, 384, 0, 1.3),
    ("tensor", 2, 257, 128, 0, 0.7),
    ("tile", 20, 48, 256, 3, 1.1),    # window longer than the 16 lanes of a row: two passes
    ("tensor", 20, 48, 256, 0, 1.1),
])
def test_sequence_bit_exact(fp8bs, mode, H, M, K, ldh_pad, growth):
    KB = K // 128
    steps = 7 if H < 16 else 24
    if mode == "tile":
        hist_d = torch.zeros(H, KB, M + ldh_pad, dtype=torch.float32, device="cuda")
    else:
        hist_d = torch.zeros(H + 2, dtype=torch.float32, device="cuda")
    stats = torch.zeros(2, dtype=torch.int32, device="cuda")
    total = np.zeros(2, np.int64)
    past = []  # the oracle's history: each step's maxima, oldest first
    for t in range(steps):
        x = synth.drifting_act(M, K, t, case=700 + H, growth=growth)
        q, s = fp8bs.fp8_quant_act_1x128_delayed(x.cuda(), hist_d, t, mode=mode, stats=stats)
        torch.cuda.synchronize()
        q_o, s_o, step_max, st = oracle.quant_act_1x128_delayed(synth.bf16_bits(x), past[-H:], mode)
        past.append(step_max)
        total += st
        gu.assert_same_bits(gu.host(q), q_o, f"{mode} step {t} codes")
        gu.assert_same_bits(gu.host(s), s_o, f"{mode} step {t} scales")
        hd = gu.host(hist_d)
        gu.assert_same_bits(hd[:, :, :M] if mode == "tile" else hd,
                            _expected_ring(past, t, H, mode, KB, M), f"{mode} step {t} ring")
        assert np.array_equal(gu.host(stats).astype(np.int64), total), (t, gu.host(stats), total)
    if growth > 1.2:
        assert total[0] > 0  # the sequences that grow do clip under delayed scaling


def test_stats_are_optional(fp8bs):
    x = synth.drifting_act(64, 256, 0, case=710)
    hist = torch.zeros(2, 2, 64, dtype=torch.float32, device="cuda")
    q, s = fp8bs.fp8_quant_act_1x128_delayed(x.cuda(), hist, 0)
    torch.cuda.synchronize()
    q0, s0 = oracle.quant_act_1x128(synth.bf16_bits(x))
    gu.assert_same_bits(gu.host(q), q0, "codes")
    gu.assert_same_bits(gu.host(s), s0, "scales")


def test_ablation_runner_small(fp8bs):
    """The online vs delayed comparison runs end to end on a small case;
    online scaling never clips, and its error is no larger than the
    delayed methods' on a growing sequence."""
    from fp8_block_scaled_05_amd import ablation
    r = ablation.run(steps=8, M=256, K=512, H=2, growths=(1.3,), timing_iters=2)
    sc = r["scenarios"]["growth_1.3"]
    assert sc["online"]["clipped_frac"] == 0.0
    assert sc["delayed_tile"]["clipped_frac"] > 0.0 and sc["delayed_tensor"]["clipped_frac"] > 0.0
    assert sc["online"]["rel_rmse"] <= min(sc["delayed_tile"]["rel_rmse"],
                                           sc["delayed_tensor"]["rel_rmse"])
    assert set(r["throughput"]) == {"online", "delayed_tile", "delayed_tensor"}
