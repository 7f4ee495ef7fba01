"""Benchmark of the block-scaled FP8 hot path on one MI355X.

One step = the whole online-FP8 linear-layer forward on the dense workload:
quantize the bf16 activations A [4096][7168] per 1x128 tile, quantize the
bf16 weights W [18432][7168] per 128x128 block (both online, from the current
values), then the block-scaled FP8 GEMM C = A.W^T with FP32 promotion every
128 K and bf16 output.  ``value`` is 2*M*N*K / (time per step), in TFLOP/s,
with all inputs resident in HBM.

The same run also times, outside the timed steps, the other workloads of the
path: the activation and weight quantizers alone at 8192x7168 / 18432x7168
(GB/s, buffers rotated past the 256 MB Infinity Cache), the grouped MoE GEMM
(32 experts, top-8 of 4096 tokens, gate/up and down), the skinny GEMM with
in-call activation quantization (M = 16, 64), the dense GEMM with its output
quantized for the next FP8 GEMM (against bf16 output followed by the
activation quantizer), the backward pass of the dense layer and of the MoE
gate/up layer (data and weight gradients with their quantizers), online
against delayed (history-based) scaling on a
drifting sequence of activations (quantization error, clipped and flushed
fractions), and the CPU oracle on a bounded sample of the dense step
(``cpu_baseline``).

The default 300 warm-up steps (about 0.2 s) bring the engine clock to its
sustained level before the timed steps; with only a few warm-up steps the
first timed GEMMs run at a lower clock.

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 300] [--no-parts]
       [--no-cpu-baseline]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("block-scaled FP8 GEMM TFLOP/s (+% MFMA peak); act-quant GB/s (+% HBM peak)")
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E

M, N, K = 4096, 18432, 7168
GEMM_KERNEL_SOURCES = ("gemm.hip", "gemm_kernel.hpp", "device.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_dense_gemm_M4096_N18432_K7168.txt")


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def _gemm_source_hash():
    h = hashlib.sha256()
    for f in GEMM_KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp8_block_scaled_05_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when it is absent or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != _gemm_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events around launches on torch's current stream (the stream the
    library launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))

    def avg_ms(self, name):
        self.torch.cuda.synchronize()
        ps = self.pairs.get(name, [])
        return sum(a.elapsed_time(b) for a, b in ps) / len(ps) if ps else float("nan")

    def med_ms(self, name):
        """Median over the calls: the per-workload figures of ``parts`` (a
        single stalled call, seen now and then on the boxes, would otherwise
        move a mean over 10-30 calls)."""
        self.torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in self.pairs.get(name, []))
        return ts[len(ts) // 2] if ts else float("nan")


def _dense_setup(torch, fp8bs, synth):
    a = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    w = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(K // 128, M, dtype=torch.float32, device="cuda")
    qw = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    return a, w, qa, sa, qw, sw, c


def _parts(torch, fp8bs, synth, dense, iters=30):
    import numpy as np

    out = {}
    tm = Timer(torch)

    # the dense GEMM with its output quantized for the next FP8 GEMM (E4M3
    # codes + 1x128 scales written by the GEMM), timed interleaved with the
    # unfused route: bf16 output, then the activation quantizer on it
    qa, sa, qw, sw = dense
    qc = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    scq = torch.empty(N // 128, M, dtype=torch.float32, device="cuda")
    cb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    qc2 = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    sc2 = torch.empty(N // 128, M, dtype=torch.float32, device="cuda")
    for i in range(iters + 5):
        f = lambda: fp8bs.fp8_block_gemm_e4m3_out(qa, sa, qw, sw, qc=qc, sc=scq)
        (tm.run("gemm_q", f) if i >= 5 else f())
        f2 = lambda: (fp8bs.fp8_block_gemm(qa, sa, qw, sw, out=cb),
                      fp8bs.fp8_quant_act_1x128(cb, qc2, sc2))
        (tm.run("gemm_then_q", f2) if i >= 5 else f2())
    ms, ms2 = tm.med_ms("gemm_q"), tm.med_ms("gemm_then_q")
    out["dense_gemm_e4m3_out_M4096_N18432_K7168"] = {
        "us": ms * 1e3, "TFLOPs": 2.0 * M * N * K / ms / 1e9,
        "frac_mfma": 2.0 * M * N * K / ms / 1e9 / PEAK_FP8_TFLOPS,
        "unfused_bf16_gemm_then_act_quant_us": ms2 * 1e3}
    del qc, scq, cb, qc2, sc2
    torch.cuda.empty_cache()

    # the dense step's operands (4096x7168 activation, 18432x7168 weight):
    # both quantized in one launch, timed interleaved with two launches
    a_s = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    w_s = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    for i in range(iters + 5):
        f = lambda: fp8bs.fp8_quant_linear(a_s, w_s, qa, sa, qw, sw)
        (tm.run("q_pair", f) if i >= 5 else f())
        f2 = lambda: (fp8bs.fp8_quant_act_1x128(a_s, qa, sa),
                      fp8bs.fp8_quant_w_128x128(w_s, qw, sw))
        (tm.run("q_two", f2) if i >= 5 else f2())
    ms, ms2 = tm.med_ms("q_pair"), tm.med_ms("q_two")
    byt = M * K * 3.03125 + N * K * (3.0 + 4.0 / 16384)
    out["quant_pair_one_launch_4096x7168_and_18432x7168"] = {
        "us": ms * 1e3, "GBps": byt / ms / 1e6, "frac_hbm": byt / ms / 1e6 / PEAK_HBM_GBPS,
        "two_launches_us": ms2 * 1e3}
    del a_s, w_s
    torch.cuda.empty_cache()

    # activation quantizer 8192x7168, 4 rotated buffer sets (712 MB)
    Mq, Kq = 8192, 7168
    xs = [synth.act(Mq, Kq, case=synth.QUANT.case_id, tensor=i, device="cuda") for i in range(4)]
    qs = [torch.empty(Mq, Kq, dtype=torch.uint8, device="cuda") for _ in range(4)]
    ss = [torch.empty(Kq // 128, Mq, dtype=torch.float32, device="cuda") for _ in range(4)]
    for i in range(iters + 5):
        j = i % 4
        f = lambda: fp8bs.fp8_quant_act_1x128(xs[j], qs[j], ss[j])
        (tm.run("qa", f) if i >= 5 else f())
    ms = tm.med_ms("qa")
    byt = Mq * Kq * 3.03125
    out["act_quant_8192x7168"] = {"us": ms * 1e3, "GBps": byt / ms / 1e6,
                                  "frac_hbm": byt / ms / 1e6 / PEAK_HBM_GBPS,
                                  "bytes": byt}

    # weight quantizer 18432x7168, 2 rotated sets (793 MB)
    ws = [synth.weight(N, K, case=synth.QUANT.case_id, tensor=10 + i, device="cuda") for i in range(2)]
    qws = [torch.empty(N, K, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sws = [torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda") for _ in range(2)]
    for i in range(iters + 5):
        j = i % 2
        f = lambda: fp8bs.fp8_quant_w_128x128(ws[j], qws[j], sws[j])
        (tm.run("qw", f) if i >= 5 else f())
    ms = tm.med_ms("qw")
    byt = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
    out["weight_quant_18432x7168"] = {"us": ms * 1e3, "GBps": byt / ms / 1e6,
                                      "frac_hbm": byt / ms / 1e6 / PEAK_HBM_GBPS, "bytes": byt}

    # the quantizer workload as a whole: the 8192x7168 activation and the
    # 18432x7168 weight in one launch, 2 rotated sets (1.15 GB)
    for i in range(iters + 5):
        j = i % 2
        f = lambda: fp8bs.fp8_quant_linear(xs[j], ws[j], qs[j], ss[j], qws[j], sws[j])
        (tm.run("qpair", f) if i >= 5 else f())
    ms = tm.med_ms("qpair")
    byt = Mq * Kq * 3.03125 + byt
    out["quant_pair_8192x7168_and_18432x7168"] = {
        "us": ms * 1e3, "GBps": byt / ms / 1e6, "frac_hbm": byt / ms / 1e6 / PEAK_HBM_GBPS,
        "bytes": byt}
    del xs, qs, ss
    torch.cuda.empty_cache()

    # skinny GEMM with in-call activation quantization, W rotated over 4 copies
    wq = [(qws[i % 2].clone(), sws[i % 2].clone()) for i in range(4)]
    del ws, qws, sws
    for Ms in (16, 64):
        x = synth.act(Ms, K, case=synth.SKINNY.case_id, tensor=Ms, device="cuda")
        cs = torch.empty(Ms, N, dtype=torch.bfloat16, device="cuda")
        sa_o = torch.empty(K // 128, Ms, dtype=torch.float32, device="cuda")
        wsp = torch.empty(fp8bs.workspace_bytes(fp8bs.OP_GEMM_BF16, Ms, N, K), dtype=torch.uint8,
                          device="cuda")
        name = f"skinny{Ms}"
        for i in range(iters + 5):
            q, s = wq[i % 4]
            f = lambda: fp8bs.fp8_block_gemm(x, sa_o, q, s, out=cs, workspace=wsp)
            (tm.run(name, f) if i >= 5 else f())
        ms = tm.med_ms(name)
        byt = N * K + (N // 128) * (K // 128) * 4 + Ms * K * 2 + Ms * N * 2
        out[f"skinny_fused_M{Ms}_N18432_K7168"] = {
            "us": ms * 1e3, "GBps": byt / ms / 1e6, "frac_hbm": byt / ms / 1e6 / PEAK_HBM_GBPS,
            "TFLOPs": 2 * Ms * N * K / ms / 1e9, "bytes": byt}
    del wq
    torch.cuda.empty_cache()

    # grouped MoE: 4096 tokens, top-8 of 32 experts; gate/up N=4096 K=7168,
    # down N=7168 K=2048; step = quantize A's and all expert weights + 2 GEMMs
    G, T = 32, 4096
    order, offsets = synth.routing(T, G, 8, case=synth.MOE.case_id)
    Mt = int(offsets[-1])
    off_d = torch.from_numpy(offsets).cuda()
    tokens = synth.act(T, 7168, case=synth.MOE.case_id, tensor=0, device="cuda")
    a1 = tokens[torch.from_numpy(order).cuda()]
    del tokens
    a2 = synth.act(Mt, 2048, case=synth.MOE.case_id, tensor=1, device="cuda")
    w1 = synth.expert_weights(G, 4096, 7168, case=synth.MOE.case_id, tensor=10, device="cuda")
    w2 = synth.expert_weights(G, 7168, 2048, case=synth.MOE.case_id, tensor=100, device="cuda")
    qa1 = torch.empty(Mt, 7168, dtype=torch.uint8, device="cuda")
    sa1 = torch.empty(56, Mt, dtype=torch.float32, device="cuda")
    qa2 = torch.empty(Mt, 2048, dtype=torch.uint8, device="cuda")
    sa2 = torch.empty(16, Mt, dtype=torch.float32, device="cuda")
    qw1 = torch.empty(G, 4096, 7168, dtype=torch.uint8, device="cuda")
    sw1 = torch.empty(G, 32, 56, dtype=torch.float32, device="cuda")
    qw2 = torch.empty(G, 7168, 2048, dtype=torch.uint8, device="cuda")
    sw2 = torch.empty(G, 56, 16, dtype=torch.float32, device="cuda")
    c1 = torch.empty(Mt, 4096, dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty(Mt, 7168, dtype=torch.bfloat16, device="cuda")

    def moe_step(timed):
        run = tm.run if timed else (lambda n, f: f())
        run("moe_qa", lambda: (fp8bs.fp8_quant_act_1x128(a1, qa1, sa1),
                               fp8bs.fp8_quant_act_1x128(a2, qa2, sa2)))
        # stacked [G*N][K] weights: 128x128 blocks never straddle experts
        run("moe_qw", lambda: (fp8bs.fp8_quant_w_128x128(w1.view(G * 4096, 7168),
                                                         qw1.view(G * 4096, 7168),
                                                         sw1.view(G * 32, 56)),
                               fp8bs.fp8_quant_w_128x128(w2.view(G * 7168, 2048),
                                                         qw2.view(G * 7168, 2048),
                                                         sw2.view(G * 56, 16))))
        run("moe_g1", lambda: fp8bs.fp8_block_grouped_gemm(qa1, sa1, qw1, sw1, off_d, out=c1))
        run("moe_g2", lambda: fp8bs.fp8_block_grouped_gemm(qa2, sa2, qw2, sw2, off_d, out=c2))

    for i in range(3):
        moe_step(False)
    for i in range(10):
        moe_step(True)
    f1 = 2.0 * Mt * 4096 * 7168
    f2 = 2.0 * Mt * 7168 * 2048
    g1, g2 = tm.med_ms("moe_g1"), tm.med_ms("moe_g2")
    tot = g1 + g2 + tm.med_ms("moe_qa") + tm.med_ms("moe_qw")
    out["moe_grouped_E32_top8_T4096"] = {
        "M_total": Mt, "experts_empty": int((offsets[1:] == offsets[:-1]).sum()),
        "gate_up_us": g1 * 1e3, "gate_up_TFLOPs": f1 / g1 / 1e9,
        "down_us": g2 * 1e3, "down_TFLOPs": f2 / g2 / 1e9,
        "gemms_TFLOPs": (f1 + f2) / (g1 + g2) / 1e9,
        "gemms_frac_mfma": (f1 + f2) / (g1 + g2) / 1e9 / PEAK_FP8_TFLOPS,
        "step_with_quant_us": tot * 1e3, "step_TFLOPs": (f1 + f2) / tot / 1e9}
    del a2, w2, qa2, sa2, qw2, sw2, c2, c1

    # MoE backward of the gate/up layer (same routing): data gradient
    # dX = dY . W_g (grouped GEMM over per-expert transposed weights) and
    # weight gradients dW_g = dY_g^T . X_g (one launch over the experts'
    # 128-padded token ranges)
    dy1 = synth.act(Mt, 4096, case=synth.MOE.case_id, tensor=2, device="cuda")
    qwt = torch.empty(G, 7168, 4096, dtype=torch.uint8, device="cuda")
    swt = torch.empty(G, 56, 32, dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8bs.fp8_quant_w_128x128_t(w1[g], qw1[g], sw1[g], qwt[g], swt[g])
    del w1, qw1, sw1
    sizes = offsets[1:] - offsets[:-1]
    poff = np.concatenate([[0], np.cumsum((sizes + 127) // 128 * 128)]).astype(np.int32)
    Tp = int(poff[-1])
    dyp = torch.zeros(Tp, 4096, dtype=torch.bfloat16, device="cuda")
    xp = torch.zeros(Tp, 7168, dtype=torch.bfloat16, device="cuda")
    for g in range(G):
        n = int(sizes[g])
        dyp[poff[g]:poff[g] + n] = dy1[offsets[g]:offsets[g] + n]
        xp[poff[g]:poff[g] + n] = a1[offsets[g]:offsets[g] + n]
    poff_d = torch.from_numpy(poff).cuda()
    qdy1 = torch.empty(Mt, 4096, dtype=torch.uint8, device="cuda")
    sdy1 = torch.empty(32, Mt, dtype=torch.float32, device="cuda")
    dx1 = torch.empty(Mt, 7168, dtype=torch.bfloat16, device="cuda")
    qdyt = torch.empty(4096, Tp, dtype=torch.uint8, device="cuda")
    sdyt = torch.empty(Tp // 128, 4096, dtype=torch.float32, device="cuda")
    qxt = torch.empty(7168, Tp, dtype=torch.uint8, device="cuda")
    sxt = torch.empty(Tp // 128, 7168, dtype=torch.float32, device="cuda")
    dw1 = torch.empty(G, 4096, 7168, dtype=torch.float32, device="cuda")
    dw1b = torch.empty(G, 4096, 7168, dtype=torch.bfloat16, device="cuda")

    def moe_bwd(timed):
        run = tm.run if timed else (lambda n, f: f())
        run("mb_q", lambda: (fp8bs.fp8_quant_act_1x128(dy1, qdy1, sdy1),
                             fp8bs.fp8_quant_act_128x1_t(dyp, qdyt, sdyt),
                             fp8bs.fp8_quant_act_128x1_t(xp, qxt, sxt)))
        run("mb_dx", lambda: fp8bs.fp8_block_grouped_gemm(qdy1, sdy1, qwt, swt, off_d, out=dx1))
        run("mb_dw", lambda: fp8bs.fp8_block_kgrouped_gemm_rowscaled(qdyt, sdyt, qxt, sxt, poff_d,
                                                                     out=dw1))
        run("mb_dw16", lambda: fp8bs.fp8_block_kgrouped_gemm_rowscaled(qdyt, sdyt, qxt, sxt,
                                                                       poff_d, out=dw1b))

    for i in range(3):
        moe_bwd(False)
    for i in range(10):
        moe_bwd(True)
    fdx = 2.0 * Mt * 4096 * 7168
    fdw = 2.0 * Tp * 4096 * 7168  # padded tokens included (zero rows)
    tdx, tdw, tq = tm.med_ms("mb_dx"), tm.med_ms("mb_dw"), tm.med_ms("mb_q")
    out["moe_backward_gate_up_E32_top8_T4096"] = {
        "tokens_padded": Tp,
        "dgrad_us": tdx * 1e3, "dgrad_TFLOPs": fdx / tdx / 1e9,
        "wgrad_us": tdw * 1e3, "wgrad_TFLOPs": fdw / tdw / 1e9,
        "wgrad_useful_TFLOPs": fdx / tdw / 1e9,
        "wgrad_bf16_out_us": tm.med_ms("mb_dw16") * 1e3,
        "wgrad_bf16_out_TFLOPs": fdw / tm.med_ms("mb_dw16") / 1e9,
        "quantizers_us": tq * 1e3}
    del dy1, qwt, swt, dyp, xp, qdy1, sdy1, dx1, qdyt, sdyt, qxt, sxt, dw1, dw1b, a1
    torch.cuda.empty_cache()

    # backward pass of the dense layer (tokens 4096, N=18432, K=7168):
    # quantizers with transposed outputs, data gradient dX = dY . W
    # (contraction 18432) and weight gradient dW = dY^T . X (contraction 4096)
    Mb = M
    dy = synth.act(Mb, N, case=synth.DENSE.case_id, tensor=20, device="cuda")
    xb = synth.act(Mb, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    wb = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    bq = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    bs = torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")
    bqt = torch.empty(K, N, dtype=torch.uint8, device="cuda")
    bst = torch.empty(K // 128, N // 128, dtype=torch.float32, device="cuda")
    qdy = torch.empty(Mb, N, dtype=torch.uint8, device="cuda")
    sdy = torch.empty(N // 128, Mb, dtype=torch.float32, device="cuda")
    qdyt = torch.empty(N, Mb, dtype=torch.uint8, device="cuda")
    sdyt = torch.empty(Mb // 128, N, dtype=torch.float32, device="cuda")
    qxt = torch.empty(K, Mb, dtype=torch.uint8, device="cuda")
    sxt = torch.empty(Mb // 128, K, dtype=torch.float32, device="cuda")
    dx = torch.empty(Mb, K, dtype=torch.bfloat16, device="cuda")
    dw = torch.empty(N, K, dtype=torch.float32, device="cuda")

    def bwd(timed):
        run = tm.run if timed else (lambda n, f: f())
        run("b_qw", lambda: fp8bs.fp8_quant_w_128x128_t(wb, bq, bs, bqt, bst))
        run("b_qdy", lambda: fp8bs.fp8_quant_act_1x128(dy, qdy, sdy))
        run("b_qdyt", lambda: fp8bs.fp8_quant_act_128x1_t(dy, qdyt, sdyt))
        run("b_qxt", lambda: fp8bs.fp8_quant_act_128x1_t(xb, qxt, sxt))
        run("b_dx", lambda: fp8bs.fp8_block_gemm(qdy, sdy, bqt, bst, out=dx))
        run("b_dw", lambda: fp8bs.fp8_block_gemm_rowscaled(qdyt, sdyt, qxt, sxt, out=dw))

    for i in range(iters + 5):
        bwd(i >= 5)
    fl = 2.0 * Mb * N * K
    t = {k: tm.med_ms(k) for k in ("b_qw", "b_qdy", "b_qdyt", "b_qxt", "b_dx", "b_dw")}
    out["backward_dense_M4096_N18432_K7168"] = {
        "weight_quant_with_transpose_us": t["b_qw"] * 1e3,
        "weight_quant_with_transpose_GBps": N * K * 4 / t["b_qw"] / 1e6,
        "dy_quant_1x128_us": t["b_qdy"] * 1e3,
        "dy_quant_128x1_t_us": t["b_qdyt"] * 1e3,
        "dy_quant_128x1_t_GBps": Mb * N * 3.03125 / t["b_qdyt"] / 1e6,
        "x_quant_128x1_t_us": t["b_qxt"] * 1e3,
        "dgrad_us": t["b_dx"] * 1e3, "dgrad_TFLOPs": fl / t["b_dx"] / 1e9,
        "dgrad_frac_mfma": fl / t["b_dx"] / 1e9 / PEAK_FP8_TFLOPS,
        "wgrad_us": t["b_dw"] * 1e3, "wgrad_TFLOPs": fl / t["b_dw"] / 1e9,
        "wgrad_frac_mfma": fl / t["b_dw"] / 1e9 / PEAK_FP8_TFLOPS,
        "step_us": sum(t.values()) * 1e3}
    del dy, xb, wb, bq, bs, bqt, bst, qdy, sdy, qdyt, sdyt, qxt, sxt, dx, dw
    torch.cuda.empty_cache()

    # online vs delayed scaling on drifting activations (quality, not speed)
    from fp8_block_scaled_05_amd import ablation
    out["online_vs_delayed_scaling_M4096_K7168"] = ablation.run(steps=24, timing_iters=10)
    return out


def _rounded(v):
    if isinstance(v, dict):
        return {k: _rounded(x) for k, x in v.items()}
    if isinstance(v, float):
        return float(f"{v:.5g}")
    return v


def _cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the dense step: the
    same N and K, 2048 of the 4096 rows of A (about 10-15 s on 16 cores)."""
    import numpy as np

    import oracle
    from fp8_block_scaled_05_amd import synth

    Ms, Ns = 2048, N
    a = synth.bf16_bits(synth.act(Ms, K, case=synth.DENSE.case_id, tensor=50))
    w = synth.bf16_bits(synth.weight(Ns, K, case=synth.DENSE.case_id, tensor=51))
    t0 = time.perf_counter()
    qa, sa = oracle.quant_act_1x128(a)
    qw, sw = oracle.quant_w_128x128(w)
    oracle.block_gemm(qa, sa, qw, sw)
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    return {"value": 2.0 * Ms * Ns * K / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"dense step (1x128 act quant, 128x128 weight quant, float64 block GEMM) "
                      f"on M={Ms}, N={Ns}, K={K}: {dt:.2f} s"}


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from fp8_block_scaled_05_amd import fp8bs, synth

    a, w, qa, sa, qw, sw, c = _dense_setup(torch, fp8bs, synth)
    tm = Timer(torch)

    def step(timed):
        run = tm.run if timed else (lambda n, f: f())
        run("quant", lambda: fp8bs.fp8_quant_linear(a, w, qa, sa, qw, sw))
        run("gemm", lambda: fp8bs.fp8_block_gemm(qa, sa, qw, sw, out=c))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12

    g_ms = tm.avg_ms("gemm")
    q_ms = tm.avg_ms("quant")
    gemm_tflops = flops / (g_ms * 1e-3) / 1e12
    traffic = _traffic()
    # algorithmic bytes of the one-launch quantizer pair: bf16 in, codes and
    # scales out, for the activation (1x128 tiles) and the weight (128x128)
    quant_bytes = M * K * 3.03125 + N * K * (3.0 + 4.0 / 16384)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 x e4m3 -> fp32 accumulate, bf16 out",
        "data": "synthetic (seeded; bf16 N(0,1) x per-row LogNormal(0,1) activations with "
                "0.1% x100 outliers, N(0,0.02) weights)",
        "config": {"workload": "dense_fp8_linear_M4096_N18432_K7168 (online 1x128 act quant + "
                               "128x128 weight quant in one launch + block-scaled GEMM, "
                               "bf16 out)",
                   "M": M, "N": N, "K": K, "group": 128},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic, "kernel": "block_gemm_kernel",
                     "kernel_us": round(g_ms * 1e3, 2)},
        "breakdown_us": {"quant_act_and_weight": round(q_ms * 1e3, 2),
                         "gemm": round(g_ms * 1e3, 2)},
        "quant_in_step": {"GBps": round(quant_bytes / q_ms / 1e6, 1),
                          "frac_hbm": round(quant_bytes / q_ms / 1e6 / PEAK_HBM_GBPS, 4)},
    }
    if not args.no_parts:
        line["parts"] = _rounded(_parts(torch, fp8bs, synth, (qa, sa, qw, sw)))
    line["cpu_baseline"] = None if args.no_cpu_baseline else _cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
