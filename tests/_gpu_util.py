"""Helpers shared by the GPU parity tests: host<->device copies of raw bits and
the element-wise GEMM tolerance check."""

import numpy as np
import torch

TOL = 2e-3  # |C_gpu - C| <= TOL * sum_k |a_k b_k| on the same quantized inputs


def dev():
    return torch.device("cuda:0")


def bf16_from_bits(bits, device=None):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device or dev())


def u8(a, device=None):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device or dev())


def f32(a, device=None):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device or dev())


def host(t):
    return t.detach().cpu().numpy()


def host_f64(t):
    return t.detach().float().cpu().double().numpy()


def check_gemm(c_gpu, C, B, tol=TOL, bf16=None):
    """Assert the tolerance on every element; return the worst ratio.

    The 2e-3 * sum|a b| bar applies to the FP32 result.  A bf16 output is
    that result rounded to nearest even, which adds at most 2^-8 of its
    magnitude (|result| <= |C| + 2e-3 * B); that rounding is allowed for.
    """
    if bf16 is None:
        bf16 = isinstance(c_gpu, torch.Tensor) and c_gpu.dtype == torch.bfloat16
    got = c_gpu if isinstance(c_gpu, np.ndarray) else host_f64(c_gpu)
    err = np.abs(got - C)
    assert np.all(np.isfinite(got)), "non-finite GEMM output"
    bound = tol * B
    if bf16:
        bound = bound + 2.0 ** -8 * (np.abs(C) + tol * B)
    zero = bound == 0
    assert np.all(err[zero] == 0), "nonzero output where the exact result is 0"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= 1.0, f"max |err| / (2e-3 * sum|ab|) = {worst}"
    return worst


def assert_same_bits(gpu, ref, what):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    if gpu.dtype == np.float32:
        gpu, ref = gpu.view(np.uint32), ref.view(np.uint32)
    bad = np.nonzero(gpu != ref)
    n = bad[0].size
    assert n == 0, f"{what}: {n} mismatches, first at {tuple(b[0] for b in bad)}: " \
                   f"gpu {gpu[tuple(b[0] for b in bad)]:#x} ref {ref[tuple(b[0] for b in bad)]:#x}"
