"""Pins of the oracle's E4M3 codec against the format definition, a library
decoder, hand-worked rounding cases and brute force."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import e4m3
from tests import _golden


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_golden_values():
    tab = oracle.decode_table()
    for code, val in _golden.e4m3_codes():
        if val == "nan":
            assert math.isnan(tab[code])
        else:
            assert tab[code] == float(val), hex(code)
            if val.startswith("-"):
                assert math.copysign(1.0, tab[code]) < 0


def test_decode_matches_library_decoder_all_codes():
    ours = oracle.decode_table()
    lib = _torch_decode_all()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_encode_decode_roundtrip_all_finite_codes():
    tab = oracle.decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert len(codes) == 254
    back = oracle.encode(tab[codes].astype(np.float32))
    assert np.array_equal(back, codes)


def test_encode_golden_rounding():
    for val, code in _golden.e4m3_rounding():
        got = int(oracle.encode(np.array([float(val)], dtype=np.float32))[0])
        assert got == code, (val, hex(got), hex(code))


def _stratified_f32(limit=448.0):
    """Every bf16-prefix (top 16 bits) of float32, combined with low halves
    that sit on, just below and just above every rounding boundary."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    f = bits.view(np.float32)
    ok = np.isfinite(f) & (np.abs(f) <= limit)
    return f[ok]


def test_encode_matches_library_rne_in_range():
    # torch's cast is round-to-nearest-even without saturation; inside
    # [-448, 448] the two must agree bit for bit.
    y = _stratified_f32()
    ours = oracle.encode(y)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != lib)[0]
    assert bad.size == 0, [(float(y[i]), hex(ours[i]), hex(lib[i])) for i in bad[:5]]


def _brute_force_encode(y):
    """argmin over all finite codes of |dec(c) - y|, ties to the even code,
    saturating, sign kept.  Pure Python per value."""
    tab = oracle.decode_table()
    out = []
    for v in np.asarray(y, dtype=np.float32).tolist():
        neg = math.copysign(1.0, v) < 0
        a = min(abs(v), 448.0)
        best = None
        for c in range(0x7F):
            d = abs(tab[c] - a)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out.append(best[1] | (0x80 if neg else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_matches_brute_force_argmin():
    rng = np.random.default_rng(7)
    y = np.concatenate([
        rng.standard_normal(1500).astype(np.float32) * np.float32(60.0),
        rng.uniform(-0.03, 0.03, 800).astype(np.float32),
        _stratified_f32()[::997],
        np.array([0.0, -0.0, 447.9, 448.0, 460.0, -470.0], dtype=np.float32),
    ]).astype(np.float32)
    assert np.array_equal(oracle.encode(y), _brute_force_encode(y))


def test_encode_monotone():
    y = np.sort(_stratified_f32())
    dec = oracle.decode(oracle.encode(y))
    assert np.all(np.diff(dec) >= 0)


def test_encode_saturates_and_keeps_sign_of_zero():
    y = np.array([1e30, -1e30, 448.0, 449.0, -0.0, -1e-30, 1e-30], dtype=np.float32)
    assert oracle.encode(y).tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x80, 0x80, 0x00]


@pytest.mark.slow
def test_encode_exhaustive_in_range():
    """Every float32 in [-448, 448] against the library cast (about 2.3e9
    values; opt-in)."""
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        bits = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        f = bits.view(np.float32)
        f = f[np.isfinite(f) & (np.abs(f) <= 448.0)]
        if f.size == 0:
            continue
        lib = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.encode(f), lib), hex(start)


def test_mutant_encoder_is_caught():
    """A plausible slip (ties away from zero instead of to even) must fail the
    golden rounding pins."""
    mid = e4m3._MID

    def mutant(y):
        y = np.asarray(y, dtype=np.float32)
        v = np.abs(y).astype(np.float64)
        lo = np.clip(np.searchsorted(e4m3._MAG, v, side="right") - 1, 0, 126)
        up = (lo < 126) & (v >= mid[np.minimum(lo, 125)])
        mag = np.where(v >= 448, 0x7E, lo + up).astype(np.uint8)
        return (mag | (np.signbit(y).astype(np.uint8) << 7)).astype(np.uint8)

    fails = 0
    for val, code in _golden.e4m3_rounding():
        if int(mutant(np.array([float(val)], dtype=np.float32))[0]) != code:
            fails += 1
    assert fails > 0
