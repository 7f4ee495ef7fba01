"""Pins of the oracle's online 1x128 / 128x128 quantizers: hand-worked tiles,
closed forms of the scale rule, the round-trip error bound, invariants and an
independent brute-force encoder."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import quant
from tests import _golden


def _bf16_bits(x):
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return quant.bf16_bits_to_f32(bits)


def _heavy_tiles(rows, k, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)) * np.exp(rng.standard_normal((rows, 1)))
    n_out = max(1, rows * k // 1000)
    idx = rng.choice(rows * k, n_out, replace=False)
    x.ravel()[idx] *= 100.0
    return _bf16_bits(x)


def test_worked_tiles():
    for name, (entries, scale_bits, codes) in _golden.quant_tiles().items():
        x = np.zeros(128, dtype=np.float32)
        for i, v in entries.items():
            x[i] = float(v)
        bits = _bf16_bits(x)
        # the fixtures use bf16-exact values only
        assert np.array_equal(_f32(bits), x) and np.array_equal(np.signbit(_f32(bits)), np.signbit(x))
        q, s = oracle.quant_act_1x128(bits[None, :])
        assert int(s[0, 0].view(np.uint32)) == scale_bits, name
        want = np.zeros(128, dtype=np.uint8)
        for i, c in codes.items():
            want[i] = c
        assert np.array_equal(q[0], want), (name, [hex(v) for v in q[0][:16]])


def _all_positive_bf16_at_least_floor():
    bits = np.arange(0x0000, 0x7F80, dtype=np.uint16)  # positive finite bf16
    f = _f32(bits)
    return f[f >= 2.0 ** -64]


def test_tile_maximum_maps_to_448_for_every_bf16_amax():
    a = _all_positive_bf16_at_least_floor()
    s, r = oracle.tile_scale(a)
    y = np.multiply(a, r, dtype=np.float32)
    assert np.all(np.abs(y.astype(np.float64) - 448.0) <= 448.0 * 2.0 ** -23)
    assert np.all(oracle.encode(y) == 0x7E)
    assert np.all(oracle.encode(-y) == 0xFE)
    # s is a/448 correctly rounded
    assert np.all(np.abs(s.astype(np.float64) * 448.0 - a) <= a.astype(np.float64) * 2.0 ** -24)
    # r is 448/a correctly rounded
    assert np.all(np.abs(r.astype(np.float64) * a - 448.0) <= 448.0 * 2.0 ** -24)


def test_argmax_element_code_on_random_tiles():
    bits = _heavy_tiles(256, 1024, seed=3)
    q, s = oracle.quant_act_1x128(bits)
    x = _f32(bits).reshape(256, 8, 128)
    qq = q.reshape(256, 8, 128)
    am = np.argmax(np.abs(x), axis=2)
    top = np.take_along_axis(qq, am[..., None], axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    assert np.array_equal(s.T, np.max(np.abs(x), axis=2).astype(np.float32) / np.float32(448.0))


def test_round_trip_error_bound():
    bits = _heavy_tiles(512, 1024, seed=4)
    x = _f32(bits).astype(np.float64)
    q, s = oracle.quant_act_1x128(bits)
    deq = oracle.decode(q) * np.repeat(s.T.astype(np.float64), 128, axis=1)
    amax = np.repeat(np.max(np.abs(x).reshape(512, 8, 128), axis=2), 128, axis=1)
    bound = np.maximum(np.abs(x) / 16.0, amax / 458752.0) * (1 + 2.0 ** -20)
    ratio = np.abs(x - deq) / bound
    assert ratio.max() <= 1.0, ratio.max()
    assert ratio.max() > 0.9  # the bound is tight, not vacuous


def test_power_of_two_scaling_invariance():
    bits = _heavy_tiles(64, 512, seed=5)
    q0, s0 = oracle.quant_act_1x128(bits)
    for j in (-3, 5):
        bits_j = _bf16_bits(_f32(bits) * np.float32(2.0 ** j))
        assert np.array_equal(_f32(bits_j), _f32(bits) * np.float32(2.0 ** j))
        qj, sj = oracle.quant_act_1x128(bits_j)
        assert np.array_equal(qj, q0)
        assert np.array_equal(sj, s0 * np.float32(2.0 ** j))


def test_negation_flips_sign_bit_only():
    bits = _heavy_tiles(64, 512, seed=6)
    q0, s0 = oracle.quant_act_1x128(bits)
    q1, s1 = oracle.quant_act_1x128(bits ^ np.uint16(0x8000))
    assert np.array_equal(q1, q0 ^ np.uint8(0x80))
    assert np.array_equal(s1, s0)


def test_permutation_within_tile_permutes_codes():
    bits = _heavy_tiles(16, 256, seed=8)
    perm = np.random.default_rng(1).permutation(128)
    pb = bits.copy()
    pb[:, :128] = bits[:, :128][:, perm]
    q0, s0 = oracle.quant_act_1x128(bits)
    q1, s1 = oracle.quant_act_1x128(pb)
    assert np.array_equal(q1[:, :128], q0[:, :128][:, perm])
    assert np.array_equal(q1[:, 128:], q0[:, 128:])
    assert np.array_equal(s1, s0)


def test_stateless_no_history():
    # Online scaling keeps no history of maxima: quantizing X2 after X1 gives
    # exactly what X2 alone gives.
    x1 = _heavy_tiles(32, 256, seed=10)
    x2 = _heavy_tiles(32, 256, seed=11)
    alone = oracle.quant_act_1x128(x2)
    oracle.quant_act_1x128(x1)
    oracle.quant_w_128x128(x1)
    after = oracle.quant_act_1x128(x2)
    assert np.array_equal(alone[0], after[0]) and np.array_equal(alone[1], after[1])


def test_codes_match_independent_argmin_encoder():
    bits = _heavy_tiles(4, 256, seed=12)
    q, s = oracle.quant_act_1x128(bits)
    x = _f32(bits)
    tab = oracle.decode_table()
    for m in range(4):
        for kb in range(2):
            t = x[m, kb * 128:(kb + 1) * 128]
            a = max(float(np.max(np.abs(t))), 2.0 ** -64)
            r = np.float32(np.float32(448.0) / np.float32(a))
            for j in range(128):
                y = float(np.float32(t[j] * r))
                mag = min(abs(y), 448.0)
                best = min(range(0x7F), key=lambda c: (abs(tab[c] - mag), c % 2))
                want = best | (0x80 if math.copysign(1.0, y) < 0 else 0)
                assert q[m, kb * 128 + j] == want


def test_zero_and_tiny_tiles_use_floor():
    x = np.zeros((2, 256), dtype=np.float32)
    x[1, 130] = 2.0 ** -100
    x[1, 5] = -0.0
    q, s = oracle.quant_act_1x128(_bf16_bits(x))
    floor_s = np.float32(2.0 ** -64) / np.float32(448.0)
    assert np.all(s == floor_s)
    assert q[1, 5] == 0x80 and q[1, 130] == 0x00 and q[0].max() == 0


def test_weight_block_equals_act_tiles_when_rows_share_amax():
    rng = np.random.default_rng(13)
    w = rng.standard_normal((256, 384)).astype(np.float32)
    # put the same maximum magnitude in every row of every 128-column group
    w = np.clip(w, -3.0, 3.0)
    w[:, ::128] = 4.0
    bits = _bf16_bits(w)
    qw, sw = oracle.quant_w_128x128(bits)
    qa, sa = oracle.quant_act_1x128(bits)
    assert np.array_equal(qw, qa)
    assert np.all(sw == sa[0, 0])


def test_weight_block_scale_and_ragged_band():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((300, 256)) * 0.02).astype(np.float32)
    bits = _bf16_bits(w)
    q, s = oracle.quant_w_128x128(bits)
    assert s.shape == (3, 2)
    x = _f32(bits)
    for nb in range(3):
        for kb in range(2):
            blk = x[nb * 128:min(300, nb * 128 + 128), kb * 128:kb * 128 + 128]
            amax = np.max(np.abs(blk))
            assert s[nb, kb] == np.float32(amax) / np.float32(448.0)
            qb = q[nb * 128:min(300, nb * 128 + 128), kb * 128:kb * 128 + 128]
            i = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert qb[i] & 0x7F == 0x7E


def test_division_form_differs_from_reciprocal_form():
    """The reading 'multiply by r = RN(448/a)' is observable: quantizing by
    dividing by s instead changes some codes, so both sides must pin it."""
    bits = _heavy_tiles(512, 1024, seed=15)
    x = _f32(bits).reshape(512, 8, 128)
    amax = np.max(np.abs(x), axis=2, keepdims=True)
    s, r = oracle.tile_scale(amax)
    by_r = oracle.encode(np.multiply(x, r, dtype=np.float32))
    by_s = oracle.encode(np.divide(x, s, dtype=np.float32))
    assert np.count_nonzero(by_r != by_s) > 0


# ---- float32-input tiles (the GEMM output quantized for the next GEMM) ----

def _f32_tiles(rows, k, seed):
    """Heavy-tailed float32 values with full 24-bit significands (not bf16)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, k)) * np.exp(rng.standard_normal((rows, 1)))
    idx = rng.choice(rows * k, max(1, rows * k // 1000), replace=False)
    x.ravel()[idx] *= 100.0
    x = x.astype(np.float32)
    # most values are not bf16-representable (the widening test would be vacuous)
    assert np.mean((x.view(np.uint32) & 0xFFFF) != 0) > 0.99
    return x


def test_rows_quantizer_equals_bf16_path_on_bf16_values():
    bits = _heavy_tiles(64, 512, seed=20)
    qa, sa = oracle.quant_act_1x128(bits)
    qr, sr = oracle.quant_rows_1x128(_f32(bits))
    assert np.array_equal(qa, qr) and np.array_equal(sa, sr)


def test_rows_quantizer_argmax_scale_and_round_trip():
    x = _f32_tiles(256, 1024, seed=21)
    q, s = oracle.quant_rows_1x128(x)
    xt = x.reshape(256, 8, 128)
    amax = np.max(np.abs(xt), axis=2)
    # scale: amax / 448 correctly rounded in float32
    assert np.array_equal(s.T, np.divide(amax, np.float32(448.0), dtype=np.float32))
    assert np.all(np.abs(s.T.astype(np.float64) * 448.0 - amax) <= amax * 2.0 ** -24)
    top = np.take_along_axis(q.reshape(256, 8, 128), np.argmax(np.abs(xt), axis=2)[..., None],
                             axis=2)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    deq = oracle.decode(q) * np.repeat(s.T.astype(np.float64), 128, axis=1)
    bound = np.maximum(np.abs(x) / 16.0, np.repeat(amax, 128, axis=1) / 458752.0) * (1 + 2.0 ** -20)
    ratio = np.abs(x.astype(np.float64) - deq) / bound
    assert ratio.max() <= 1.0 and ratio.max() > 0.9


def test_rows_quantizer_top_code_for_random_float32_maxima():
    # the scale rule maps any float32 maximum (not only bf16 ones) to 448
    rng = np.random.default_rng(22)
    a = np.exp2(rng.uniform(-60, 100, 200000)).astype(np.float32)
    s, r = oracle.tile_scale(a)
    y = np.multiply(a, r, dtype=np.float32)
    assert np.all(np.abs(y.astype(np.float64) - 448.0) <= 448.0 * 2.0 ** -22)
    assert np.all(oracle.encode(y) == 0x7E)


def test_rows_quantizer_matches_argmin_encoder():
    x = _f32_tiles(4, 256, seed=23)
    q, s = oracle.quant_rows_1x128(x)
    tab = oracle.decode_table()
    for m in range(4):
        for kb in range(2):
            t = x[m, kb * 128:(kb + 1) * 128]
            a = max(float(np.max(np.abs(t))), 2.0 ** -64)
            r = np.float32(np.float32(448.0) / np.float32(a))
            for j in range(128):
                y = float(np.float32(t[j] * r))
                mag = min(abs(y), 448.0)
                best = min(range(0x7F), key=lambda c: (abs(tab[c] - mag), c % 2))
                assert q[m, kb * 128 + j] == best | (0x80 if math.copysign(1.0, y) < 0 else 0)
