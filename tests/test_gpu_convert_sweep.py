"""Exhaustive parity of the device E4M3 convert (the encoder of the single
FP8 format: "Advantages of using FP8 for GEMM operations in DeepSeek-V3",
item 6): every non-NaN float32 value, both signs, zero to infinity (4.28e9
inputs), goes through the library's own ``cvt2_e4m3`` (clamp to +-448, then
the gfx950 round-to-nearest-even convert) in a test-only kernel, and must
give the oracle encoder's code.

The codes of one sign, taken in bit-pattern order, change only where the
rounded magnitude does.  The oracle's change points come from bisection over
bit patterns with ``oracle.encode``, which is monotone in the magnitude (a
property pinned by ``test_oracle_e4m3``).  The GPU codes are walked in chunks
of 2^28 consecutive patterns; equal change points and an equal code on every
run mean that all 4.28e9 codes equal the oracle's.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "libconvert_sweep.so")
LAST = 0x7F800000   # +infinity: the largest non-NaN magnitude pattern
CHUNK = 1 << 28


def _enc_bits(b):
    return int(oracle.encode(np.array([b], dtype=np.uint32).view(np.float32))[0])


def _oracle_change_points(sign):
    """First bit pattern (offset from the sign's base) of each magnitude code
    1..0x7E, found by bisection; the code of pattern 0 is 0x00 | sign."""
    base = sign << 31
    pts = []
    for c in range(1, 0x7F):
        lo, hi = 0, LAST          # enc(base + hi) & 0x7F >= c, enc(base + 0) & 0x7F < c
        assert _enc_bits(base + hi) & 0x7F >= c and _enc_bits(base) & 0x7F < c
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if _enc_bits(base + mid) & 0x7F >= c:
                hi = mid
            else:
                lo = mid
        pts.append(hi)
    return pts


def _lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run python -m fp8_block_scaled_05_amd.build")
    lib = ctypes.CDLL(LIB)
    lib.fp8bs_test_convert_range.restype = ctypes.c_int
    lib.fp8bs_test_convert_range.argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("sign", [0, 1])
def test_every_float32_value(sign):
    lib = _lib()
    base = sign << 31
    stream = torch.cuda.current_stream().cuda_stream
    codes = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    starts, values = [0], []
    prev = None
    total = LAST + 1
    for s0 in range(0, total, CHUNK):
        n = min(CHUNK, total - s0)
        st = lib.fp8bs_test_convert_range(base + s0, n, codes.data_ptr(), 0, stream)
        assert st == 0, f"launch status {st}"
        c = codes[:n]
        first = int(c[0])
        if prev is None:
            values.append(first)
        elif first != prev:
            starts.append(s0)
            values.append(first)
        chg = torch.nonzero(c[1:] != c[:-1]).flatten() + 1
        if chg.numel():
            starts.extend((chg + s0).tolist())
            values.extend(c[chg].tolist())
        prev = int(c[n - 1])
    torch.cuda.synchronize()
    want_starts = [0] + _oracle_change_points(sign)
    want_values = [(sign << 7) | m for m in range(0x7F)]
    assert len(starts) == len(want_starts), f"{len(starts)} runs, oracle {len(want_starts)}"
    bad = [i for i in range(len(starts))
           if starts[i] != want_starts[i] or values[i] != want_values[i]]
    assert not bad, (f"first mismatch at run {bad[0]}: gpu starts at {starts[bad[0]]:#x} with "
                     f"{values[bad[0]]:#x}, oracle {want_starts[bad[0]]:#x} with "
                     f"{want_values[bad[0]]:#x}")


@pytest.mark.parametrize("sign", [0, 1])
def test_bare_convert_rounds_448_to_464_down(sign):
    """The few-row GEMM's in-kernel activation quantizer converts without the
    clamp to +-448.  For finite inputs the scaled value never exceeds
    448.0000534 (every bf16 tile maximum: test_oracle_quant), so that is exact
    when the bare convert takes every float32 in [448, 464) -- all 2^19 of
    them -- to the code of 448, as the oracle does (round to nearest even:
    464 is the midpoint to the first value past the format)."""
    lib = _lib()
    first, n = (sign << 31) | 0x43E00000, 0x43E80000 - 0x43E00000   # 448.0 .. 464.0 exclusive
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    st = lib.fp8bs_test_convert_range(first, n, codes.data_ptr(), 1,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"launch status {st}"
    got = codes.cpu().numpy()
    want = oracle.encode(np.arange(first, first + n, dtype=np.uint32).view(np.float32))
    assert np.all(want == ((sign << 7) | 0x7E))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} codes differ, first at {first + bad[0]:#x}: {got[bad[0]]:#x}"


def _bf16_patterns():
    """float32 bit patterns where bf16 rounding has its cases: for every
    exponent below the NaN/Inf one (subnormals included) and both signs,
    three settings of the 7 mantissa bits that bf16 keeps (0, 0x40, 0x7F,
    so that rounding up carries into the exponent and, at the largest
    exponent, past the largest finite bf16), each with all 2^16 settings of
    the 16 bits that are rounded away (ties to even included)."""
    low = np.arange(1 << 16, dtype=np.uint32)
    out = []
    for sign in (0, 1):
        for e in range(255):
            for mhi in (0x00, 0x40, 0x7F):
                out.append((sign << 31) | (e << 23) | (mhi << 16) | low)
    return np.concatenate(out)


def test_bf16_output_rounding_matches_cpu_round_to_nearest_even():
    """The GEMM epilogues write bf16 through gfx950's V_CVT_PK_BF16_F32
    (device.hpp bf16x2_rne, f32_to_bf16_rne).  Every pattern of
    _bf16_patterns (100M float32 values, plus an odd tail through the
    single-value form) must give the bf16 that torch's CPU conversion
    (round to nearest, ties to even) gives."""
    lib = _lib()
    lib.fp8bs_test_bf16_convert.restype = ctypes.c_int
    lib.fp8bs_test_bf16_convert.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p]
    pats = np.concatenate([_bf16_patterns(), np.array([0x3F808000, 0x00008000, 0x7F7FFFFF],
                                                      dtype=np.uint32)])
    assert pats.size % 2 == 1
    x = torch.from_numpy(pats.view(np.int32)).to("cuda")
    out = torch.empty(pats.size, dtype=torch.int16, device="cuda")
    st = lib.fp8bs_test_bf16_convert(x.data_ptr(), pats.size, out.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert st == 0, f"launch status {st}"
    got = out.cpu().numpy().view(np.uint16)
    want = (torch.from_numpy(pats.view(np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{bad.size} of {pats.size} differ, first input {pats[bad[0]]:#010x}: "
                           f"gpu {got[bad[0]]:#06x}, cpu {want[bad[0]]:#06x}")
