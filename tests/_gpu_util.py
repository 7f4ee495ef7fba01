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
    """Assert the tolerance on every element; return the worst ratio of the
    error to the bare bound, max |C_gpu - C| / (2e-3 * B).

    The 2e-3 * sum|a b| bar applies to the FP32 result and is asserted as it
    stands on every element of an fp32 output.  A bf16 output is that result
    rounded to nearest even, which adds up to 2^-8 of its magnitude; that
    rounding alone exceeds 2e-3 * B only where |C| > 0.5 * B
    (2^-8 * 0.5 < 2e-3).  Only on those elements (small K, a few dominant
    products) is the rounding, 2^-8 * (|C| + 2e-3 * B), added to the bound;
    every other element of a bf16 output meets the bare bar.
    """
    if bf16 is None:
        bf16 = isinstance(c_gpu, torch.Tensor) and c_gpu.dtype == torch.bfloat16
    got = c_gpu if isinstance(c_gpu, np.ndarray) else host_f64(c_gpu)
    err = np.abs(got - C)
    assert np.all(np.isfinite(got)), "non-finite GEMM output"
    bare = tol * B
    zero = bare == 0
    assert np.all(err[zero] == 0), "nonzero output where the exact result is 0"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bare))
    widened = np.zeros(ratio.shape, dtype=bool)
    if bf16:
        widened = np.abs(C) > 0.5 * B
        bound = bare + 2.0 ** -8 * (np.abs(C) + bare)
        wr = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
        assert float(wr[widened].max(initial=0.0)) <= 1.0, \
            f"bf16 output with |C| > 0.5 B: max err / (bare + rounding) = {wr[widened].max()}"
    strict = ratio[~widened]
    worst = float(strict.max()) if strict.size else 0.0
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


def oracle_map(fn, arrays, workers=None):
    """``[fn(a) for a in arrays]`` over a pool of spawned CPU processes (the
    oracle is single-threaded NumPy; full-size parity samples quantize up to
    ~1e9 weight elements).  The workers import only the oracle and NumPy and
    never touch the GPU."""
    import concurrent.futures
    import multiprocessing
    import os

    n = len(arrays)
    if n <= 1:
        return [fn(a) for a in arrays]
    workers = workers or min(16, len(os.sched_getaffinity(0)), n)
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers, mp_context=ctx) as ex:
        return list(ex.map(fn, arrays))


def report(what, ratio):
    """Print a full-size parity result (err / bare bound) on its own line."""
    print(f"\n[parity] {what}: max |err| / (2e-3 * sum|ab|) = {ratio:.4f}", flush=True)
