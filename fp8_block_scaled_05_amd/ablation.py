"""Online vs delayed scaling on drifting activations (measurement, one GPU).

The pages ("How online quantization in DeepSeek-V3 differs from delayed
quantization", items 2-4) claim that scaling each 1x128 tile from its current
values is more accurate than delayed scaling from a history of earlier
maxima, because the distribution moves during training; they give no
numbers.  This runs both on the same seeded sequence of activation tensors
(``synth.drifting_act``: a fresh draw per step, so the 0.1% x100 outliers move,
times ``growth ** step``) and reports, per method, averaged over the steps
after the history has filled:

* ``rel_rmse``: ||dec(q) * s - x|| / ||x|| (the quantization error);
* ``clipped_frac``: values that saturation changed (|x r| > 464);
* ``flushed_frac``: non-zero values quantized to a zero code;
* the kernels' throughput at this size.

Every quantization runs in the library's kernels; this module only
generates inputs and measures (dequantizing with torch's E4M3 decode).

Usage: python -m fp8_block_scaled_05_amd.ablation [--steps 24] [--M 4096] [--K 7168]
"""

import argparse
import json

import torch

from . import fp8bs, synth

CASE = 6


def _error(x, q, s):
    M, K = x.shape
    deq = q.view(torch.float8_e4m3fn).float().view(M, K // 128, 128) * s.t().unsqueeze(2)
    xf = x.float()
    err = (deq.view(M, K) - xf).square().sum().sqrt() / xf.square().sum().sqrt()
    flushed = ((xf != 0) & ((q & 0x7F) == 0)).sum()
    return float(err), int(flushed)


def run(steps=24, M=4096, K=7168, H=16, growths=(1.0, 1.05), timing_iters=20):
    dev = "cuda"
    KB = K // 128
    out = {"M": M, "K": K, "H": H, "steps": steps, "averaged_over_steps": f"{H}..{steps - 1}",
           "scenarios": {}}
    for g in growths:
        methods = {"online": None,
                   "delayed_tile": torch.zeros(H, KB, M, dtype=torch.float32, device=dev),
                   "delayed_tensor": torch.zeros(H + 2, dtype=torch.float32, device=dev)}
        acc = {k: {"rel_rmse": 0.0, "clipped": 0, "flushed": 0, "n": 0} for k in methods}
        stats = {k: torch.zeros(2, dtype=torch.int32, device=dev) for k in methods}
        for t in range(steps):
            x = synth.drifting_act(M, K, t, case=CASE, growth=g, device=dev)
            for name, hist in methods.items():
                before = stats[name].clone()
                if hist is None:
                    q, s = fp8bs.fp8_quant_act_1x128(x)
                else:
                    q, s = fp8bs.fp8_quant_act_1x128_delayed(
                        x, hist, t, mode=name.split("_")[1], stats=stats[name])
                if t < H:
                    continue
                err, flushed = _error(x, q, s)
                a = acc[name]
                a["rel_rmse"] += err
                a["flushed"] += flushed
                a["clipped"] += int((stats[name] - before)[0])
                a["n"] += 1
        res = {}
        for name, a in acc.items():
            n = max(a["n"], 1)
            res[name] = {"rel_rmse": a["rel_rmse"] / n,
                         "clipped_frac": a["clipped"] / (n * M * K),
                         "flushed_frac": a["flushed"] / (n * M * K)}
        out["scenarios"][f"growth_{g}"] = res

    # throughput of the three quantizers on one tensor (the ring persists)
    x = synth.drifting_act(M, K, 0, case=CASE, device=dev)
    q = torch.empty(M, K, dtype=torch.uint8, device=dev)
    s = torch.empty(KB, M, dtype=torch.float32, device=dev)
    ht = torch.zeros(H, KB, M, dtype=torch.float32, device=dev)
    hn = torch.zeros(H + 2, dtype=torch.float32, device=dev)
    calls = {"online": lambda t: fp8bs.fp8_quant_act_1x128(x, q, s),
             "delayed_tile": lambda t: fp8bs.fp8_quant_act_1x128_delayed(x, ht, t, "tile", q, s),
             "delayed_tensor": lambda t: fp8bs.fp8_quant_act_1x128_delayed(x, hn, t, "tensor", q, s)}
    thr = {}
    for name, f in calls.items():
        for t in range(5):
            f(t)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(5, 5 + timing_iters):
            f(t)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / timing_iters
        # bytes the method must move: x, codes, scales, plus the history it reads/writes
        byt = M * K * 3 + M * KB * 4
        if name == "delayed_tile":
            byt += (H + 1) * KB * M * 4
        thr[name] = {"us": us, "GBps": byt / us / 1e3}
    out["throughput"] = thr
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--M", type=int, default=4096)
    ap.add_argument("--K", type=int, default=7168)
    ap.add_argument("--H", type=int, default=16)
    a = ap.parse_args()
    print(json.dumps(run(a.steps, a.M, a.K, a.H), indent=1))


if __name__ == "__main__":
    main()
