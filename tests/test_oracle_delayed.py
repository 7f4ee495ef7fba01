"""Pins of the oracle's delayed (history-based) scaling: reductions to online
scaling, hand-computed saturation and flush counts, and the scale windows of
both granularities step by step."""

import numpy as np
import pytest
import torch

import oracle
from oracle import quant


def _bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _heavy(M, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))
    idx = rng.choice(M * K, max(1, M * K // 1000), replace=False)
    x.ravel()[idx] *= 100.0
    return _bits(x)


@pytest.mark.parametrize("mode,H", [("tile", 1), ("tile", 4), ("tensor", 1), ("tensor", 3)])
def test_empty_history_is_online(mode, H):
    """No history yet (an empty window, or a window of zeros) scales online."""
    bits = _heavy(40, 384, seed=1)
    zeros = [np.zeros((3, 40), np.float32) if mode == "tile" else 0.0 for _ in range(H)]
    q0, s0 = oracle.quant_act_1x128(bits)
    for window in ([], zeros):
        q, s, _, _ = oracle.quant_act_1x128_delayed(bits, window, mode=mode)
        assert np.array_equal(q, q0) and np.array_equal(s, s0)


def test_tile_history_of_the_current_maxima_is_online():
    bits = _heavy(33, 256, seed=2)
    x = quant.bf16_bits_to_f32(bits)
    cur = np.max(np.abs(x).reshape(33, 2, 128), axis=2).T.astype(np.float32)
    q, s, step_max, stats = oracle.quant_act_1x128_delayed(bits, [cur], mode="tile")
    q0, s0 = oracle.quant_act_1x128(bits)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    assert stats == (0, int(np.count_nonzero((x != 0) & ((q0 & 0x7F) == 0))))
    assert np.array_equal(step_max, cur)


def test_saturation_count_by_hand():
    # ramp x_j = j/128 (j = 1..128), history maximum 0.5: r = 896 and
    # y_j = 7 j exactly.  Clipped: 7 j > 464 <=> j >= 67 -> 62 values.
    # Codes: y >= 432 (midpoint of 416 and 448) <=> j >= 62 gives 0x7E;
    # j = 61 (y = 427) gives 416 = 0x7D.
    x = np.arange(1, 129, dtype=np.float32)[None, :] / 128.0
    window = [np.full((1, 1), 0.5, np.float32), np.full((1, 1), 0.25, np.float32)]
    q, s, _, (sat, flushed) = oracle.quant_act_1x128_delayed(_bits(x), window, mode="tile")
    assert s[0, 0] == np.float32(0.5) / np.float32(448.0)
    assert sat == 62 and flushed == 0
    assert np.all(q[0, 61:] == 0x7E) and q[0, 60] == 0x7D


def test_flush_count_by_hand():
    # current values 1.0, history maximum 2^30: x * r = 448 * 2^-30, below half
    # the smallest subnormal (2^-10) -> every value becomes a zero code
    x = np.ones((1, 128), np.float32)
    x[0, 5] = -1.0
    window = [np.full((1, 1), 2.0 ** 30, np.float32)]
    q, _, _, (sat, flushed) = oracle.quant_act_1x128_delayed(_bits(x), window, mode="tile")
    assert sat == 0 and flushed == 128
    assert np.all((q & 0x7F) == 0) and q[0, 5] == 0x80


def test_tile_window_over_steps():
    """Step u's tensor is constant (u + 1) * c_tile; with H = 2 the scale at
    step t >= 2 comes from step t - 1 (the larger of t - 2, t - 1)."""
    H, M, K = 2, 3, 256
    c = np.array([[1.0, 2.0], [0.5, 4.0], [3.0, 0.25]], np.float32)  # [M][KB]
    past = []
    for t in range(6):
        x = np.repeat(c * (t + 1), 128, axis=1)
        q, s, step_max, (sat, _) = oracle.quant_act_1x128_delayed(_bits(x), past[-H:], mode="tile")
        prev = (t if t >= 1 else t + 1)  # window maximum = step t-1's value; step 0: online
        want = np.divide((c * prev).T.astype(np.float32), np.float32(448.0), dtype=np.float32)
        assert np.array_equal(s, want), t
        # the values grew since the window by (t+1)/t >= 1.2 > 464/448: every
        # value of the tile's constant rows is clipped
        assert sat == (M * K if t >= 1 else 0), t
        assert np.array_equal(step_max, (c * (t + 1)).T)
        past.append(step_max)


def test_tensor_window():
    """Per-tensor history, H = 2: step u has tensor maximum m_u; step t's
    scale comes from max(m_{t-2}, m_{t-1}) for every tile, and the step
    reports its own tensor maximum m_t."""
    H = 2
    m = [3.0, 1.0, 0.5, 8.0, 2.0, 4.0, 1.0]
    past = []
    rng = np.random.default_rng(5)
    for t, mt in enumerate(m):
        x = rng.uniform(-1, 1, (4, 256)).astype(np.float32) * 0.5 * mt
        x[1, 7] = mt  # the tensor maximum
        bits = _bits(x)
        q, s, step_max, _ = oracle.quant_act_1x128_delayed(bits, past[-H:], mode="tensor")
        window = [m[u] for u in (t - 2, t - 1) if u >= 0]
        if window:
            assert np.all(s == np.float32(max(window)) / np.float32(448.0)), t
        else:
            q0, s0 = oracle.quant_act_1x128(bits)
            assert np.array_equal(s, s0)
        assert step_max == np.float32(mt)
        past.append(step_max)


def test_codes_follow_the_scale_rule():
    """With any window maximum, codes are the stale reciprocal's rounding:
    an independent recomputation tile by tile."""
    bits = _heavy(8, 256, seed=6)
    x = quant.bf16_bits_to_f32(bits)
    hist = np.abs(np.random.default_rng(7).standard_normal((3, 2, 8))).astype(np.float32) * 3
    q, s, _, (sat, flushed) = oracle.quant_act_1x128_delayed(bits, list(hist), mode="tile")
    n_sat = 0
    for m in range(8):
        for kb in range(2):
            a = max(float(hist[:, kb, m].max()), 2.0 ** -64)
            r = np.float32(np.float32(448.0) / np.float32(a))
            assert s[kb, m] == np.float32(np.float32(a) / np.float32(448.0))
            y = (x[m, kb * 128:(kb + 1) * 128] * r).astype(np.float32)
            n_sat += int(np.sum(np.abs(y) > 464.0))
            assert np.array_equal(q[m, kb * 128:(kb + 1) * 128],
                                  oracle.encode(np.clip(y, -448.0, 448.0)))
    assert sat == n_sat > 0
