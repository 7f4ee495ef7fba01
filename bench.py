"""Benchmark of the block-scaled FP8 hot path on one MI355X.

One step = the whole online-FP8 linear-layer forward on the dense workload:
quantize the bf16 activations A [4096][7168] per 1x128 tile, quantize the
bf16 weights W [18432][7168] per 128x128 block (both online, from the current
values, in one launch), then the block-scaled FP8 GEMM C = A.W^T with FP32
promotion every 128 K and bf16 output.  ``value`` is 2*M*N*K / (time per
step), in TFLOP/s, with all inputs resident in HBM.

The same run also times, outside the timed steps, the other workloads of the
path (``parts``): the activation and weight quantizers alone at 8192x7168 /
18432x7168 (GB/s, buffers rotated past the 256 MB Infinity Cache) and in one
launch, a plain HBM copy of the activation quantizer's byte count (the
streaming reference), the skinny GEMM with bf16 A (M = 16, 64; weights
rotated), the grouped MoE GEMM (32 experts, top-8 of 4096 tokens, gate/up and
down), the dense GEMM with its output quantized for the next FP8 GEMM, the
backward pass of the dense layer and of the MoE gate/up layer, online against
delayed scaling, and the CPU oracle (``cpu_baseline``).

Before the W warm-up steps, the step runs until 0.3 s have passed, so that
the engine clock has settled at the level it holds under this load when the
timed steps start (with a few warm-up steps alone the first GEMMs run at a
lower clock).  The line reports the engine clock of each XCD averaged over
the timed steps, from cycle-counter and wall-clock stamps taken on the GPU
just before and after them (tests/native/clock_probe.hip).

Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 300] [--no-parts]
       [--no-cpu-baseline]
       python bench.py --only PART [--iters N]   (one workload, for profiling)
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic_dense_gemm.txt")
CLOCK_SETTLE_S = 0.3


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help="run one part: " + ", ".join(PARTS))
    ap.add_argument("--iters", type=int, default=30)
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


class ClockStamps:
    """Average engine clock of each XCD over a stretch of GPU work, from the
    cycle counter and the constant-rate wall clock that a small kernel stamps
    before and after it (tests/native/clock_probe.hip: clock64 counts at the
    XCD's engine clock, wall_clock64 at the rate the runtime reports).  The
    firmware metrics that SMI tools read lag the load by about 0.4 s, longer
    than the timed steps.  Without the helper library the line carries null."""

    BLOCKS = 2048  # 8 per compute unit, so that both stamps reach every one
    LIB = os.path.join(ROOT, "tests", "native", "libclock_probe.so")

    def __init__(self, torch):
        import ctypes

        self.torch = torch
        self.lib = None
        if os.path.exists(self.LIB):
            lib = ctypes.CDLL(self.LIB)
            lib.fp8bs_clock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            lib.fp8bs_clock_stamp.restype = ctypes.c_int
            lib.fp8bs_wall_clock_khz.restype = ctypes.c_int
            self.khz = lib.fp8bs_wall_clock_khz()
            if self.khz > 0:
                self.lib = lib
        self.bufs = [torch.zeros(3 * self.BLOCKS, dtype=torch.int64, device="cuda")
                     for _ in range(2)]

    def stamp(self, i):
        if self.lib is not None:
            st = self.torch.cuda.current_stream().cuda_stream
            if self.lib.fp8bs_clock_stamp(self.bufs[i].data_ptr(), self.BLOCKS, st) != 0:
                self.lib = None

    def mhz(self):
        """{xcc: MHz}, the median over the XCD's compute units of each unit's
        cycles / wall time between its earliest stamp in launch 0 and its
        latest in launch 1; None without the helper."""
        if self.lib is None:
            return None
        self.torch.cuda.synchronize()
        first, last = {}, {}
        for key, cyc, wall in self.bufs[0].view(self.BLOCKS, 3).cpu().tolist():
            if key not in first or wall < first[key][1]:
                first[key] = (cyc, wall)
        for key, cyc, wall in self.bufs[1].view(self.BLOCKS, 3).cpu().tolist():
            if key not in last or wall > last[key][1]:
                last[key] = (cyc, wall)
        per_xcc = {}
        for key in first.keys() & last.keys():
            (c0, w0), (c1, w1) = first[key], last[key]
            if w1 > w0:
                per_xcc.setdefault(key // 256, []).append((c1 - c0) / (w1 - w0) * self.khz / 1e3)
        return {x: sorted(v)[len(v) // 2] for x, v in sorted(per_xcc.items())} or None


def _smi_snapshot():
    """Memory clock (MHz) and socket power (W) from the SMI metrics table, or
    None.  The table lags the load by about 0.4 s, so a snapshot taken right
    after the timed steps describes the settle, warm-up and timed steps."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        m = amdsmi.amdsmi_get_gpu_metrics_info(amdsmi.amdsmi_get_processor_handles()[0])
        out = {}
        for key, name in (("current_uclk", "mclk_mhz"), ("current_socket_power", "socket_power_w"),
                          ("average_socket_power", "socket_power_avg_w")):
            v = m.get(key)
            if isinstance(v, (int, float)) and 0 < v < 100000:
                out[name] = v
        return out or None
    except Exception:
        return None


def _timeit(torch, fn, iters, warm=5):
    """Median and p10/p90 (ms) of ``iters`` calls of fn(i) after ``warm``."""
    tm = Timer(torch)
    for i in range(warm):
        fn(i)
    for i in range(iters):
        tm.run("x", lambda: fn(i))
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in tm.pairs["x"])
    return ts[len(ts) // 2], ts[len(ts) // 10], ts[(len(ts) * 9) // 10]


def _streamed(torch, fn, iters, warm=5):
    """Milliseconds per call of ``iters`` back-to-back calls of fn(i) between
    one pair of events on the stream (the per-call events of _timeit add
    their own packets between the kernels)."""
    for i in range(warm):
        fn(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _streamed_rate(torch, fn, iters, byt):
    ms = _streamed(torch, fn, iters)
    return {"streamed_us": ms * 1e3, "streamed_GBps": byt / ms / 1e6,
            "streamed_frac_hbm": byt / ms / 1e6 / PEAK_HBM_GBPS}


def _rate(byt, ms):
    gbps = byt / ms / 1e6
    return {"GBps": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS}


def _flops_rate(fl, ms):
    tf = fl / ms / 1e9
    return {"TFLOPs": tf, "frac_mfma": tf / PEAK_FP8_TFLOPS}


# --------------------------------------------------------------------------
# Parts: one workload each.  part(ctx, iters) -> dict.  ``ctx`` holds torch,
# the binding and the input generator.


def part_act_quant(c, iters):
    """Activation quantizer 8192x7168, 4 rotated buffer sets (712 MB)."""
    torch, fp8bs, synth = c
    Mq, Kq = 8192, 7168
    xs = [synth.act(Mq, Kq, case=synth.QUANT.case_id, tensor=i, device="cuda") for i in range(4)]
    qs = [torch.empty(Mq, Kq, dtype=torch.uint8, device="cuda") for _ in range(4)]
    ss = [torch.empty(Kq // 128, Mq, dtype=torch.float32, device="cuda") for _ in range(4)]
    call = lambda i: fp8bs.fp8_quant_act_1x128(xs[i % 4], qs[i % 4], ss[i % 4])
    med, p10, p90 = _timeit(torch, call, iters)
    byt = Mq * Kq * 3.03125
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3, **_rate(byt, med),
            "bytes": byt, **_streamed_rate(torch, call, iters, byt)}


def part_hbm_copy(c, iters):
    """The streaming reference: torch copy_ of 88,997,888 bytes (4 rotated
    pairs), which reads and writes the activation quantizer's 177,995,776
    bytes of HBM traffic in total."""
    torch, fp8bs, synth = c
    n = 8192 * 7168 * 3.03125 / 2
    n = int(n) // 16 * 16
    src = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i) for i in range(4)]
    dst = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(4)]
    call = lambda i: dst[i % 4].copy_(src[i % 4])
    med, p10, p90 = _timeit(torch, call, iters)
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3, **_rate(2 * n, med),
            "bytes": 2 * n, **_streamed_rate(torch, call, iters, 2 * n)}


def part_weight_quant(c, iters):
    """Weight quantizer 18432x7168, 2 rotated sets (793 MB)."""
    torch, fp8bs, synth = c
    ws = [synth.weight(N, K, case=synth.QUANT.case_id, tensor=10 + i, device="cuda")
          for i in range(2)]
    qws = [torch.empty(N, K, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sws = [torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda") for _ in range(2)]
    call = lambda i: fp8bs.fp8_quant_w_128x128(ws[i % 2], qws[i % 2], sws[i % 2])
    med, p10, p90 = _timeit(torch, call, iters)
    byt = N * K * 2 + N * K + (N // 128) * (K // 128) * 4
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3, **_rate(byt, med),
            "bytes": byt, **_streamed_rate(torch, call, iters, byt)}


def part_quant_pair(c, iters):
    """The quantizer workload as a whole: the 8192x7168 activation and the
    18432x7168 weight in one launch, 2 rotated sets (1.15 GB)."""
    torch, fp8bs, synth = c
    Mq = 8192
    xs = [synth.act(Mq, K, case=synth.QUANT.case_id, tensor=i, device="cuda") for i in range(2)]
    ws = [synth.weight(N, K, case=synth.QUANT.case_id, tensor=10 + i, device="cuda")
          for i in range(2)]
    out = [(torch.empty(Mq, K, dtype=torch.uint8, device="cuda"),
            torch.empty(K // 128, Mq, dtype=torch.float32, device="cuda"),
            torch.empty(N, K, dtype=torch.uint8, device="cuda"),
            torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")) for _ in range(2)]
    call = lambda i: fp8bs.fp8_quant_linear(xs[i % 2], ws[i % 2], *out[i % 2])
    med, p10, p90 = _timeit(torch, call, iters)
    byt = Mq * K * 3.03125 + N * K * 2 + N * K + (N // 128) * (K // 128) * 4
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3, **_rate(byt, med),
            "bytes": byt, **_streamed_rate(torch, call, iters, byt)}


def _skinny(c, iters, Ms):
    torch, fp8bs, synth = c
    w = synth.weight(N, K, case=synth.SKINNY.case_id, tensor=1, device="cuda")
    qw, sw = fp8bs.fp8_quant_w_128x128(w)
    del w
    wq = [(qw.clone(), sw.clone()) for _ in range(4)]  # 4 rotated copies: 529 MB
    x = synth.act(Ms, K, case=synth.SKINNY.case_id, tensor=Ms, device="cuda")
    cs = torch.empty(Ms, N, dtype=torch.bfloat16, device="cuda")
    sa_o = torch.empty(K // 128, Ms, dtype=torch.float32, device="cuda")
    wsp = torch.empty(fp8bs.workspace_bytes(fp8bs.OP_GEMM_BF16, Ms, N, K), dtype=torch.uint8,
                      device="cuda")
    call = lambda i: fp8bs.fp8_block_gemm(x, sa_o, wq[i % 4][0], wq[i % 4][1], out=cs,
                                          workspace=wsp)
    med, p10, p90 = _timeit(torch, call, iters)
    byt = N * K + (N // 128) * (K // 128) * 4 + Ms * K * 2 + Ms * N * 2
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3, **_rate(byt, med),
            "TFLOPs": 2 * Ms * N * K / med / 1e9, "bytes": byt,
            **_streamed_rate(torch, call, iters, byt),
            "activation_quantized": "inside the GEMM kernel" if Ms <= 16 else
            "by a separate launch before the GEMM"}


def part_skinny16(c, iters):
    """Skinny GEMM, bf16 A M=16 quantized inside the GEMM kernel."""
    return _skinny(c, iters, 16)


def part_skinny64(c, iters):
    """Skinny GEMM, bf16 A M=64 (quantizer launch, then the few-row GEMM)."""
    return _skinny(c, iters, 64)


def part_dense_gemm(c, iters):
    """The dense GEMM 4096x18432x7168 alone (bf16 out), the step's operands."""
    torch, fp8bs, synth = c
    a = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    w = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    qa, sa, qw, sw = fp8bs.fp8_quant_linear(a, w)
    del a, w
    out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    med, p10, p90 = _timeit(torch, lambda i: fp8bs.fp8_block_gemm(qa, sa, qw, sw, out=out), iters,
                            warm=50)
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3,
            **_flops_rate(2.0 * M * N * K, med)}


def part_e4m3_out(c, iters):
    """The dense GEMM with E4M3 output (the next layer's input), timed
    interleaved with the unfused route: bf16 output, then the activation
    quantizer on it."""
    torch, fp8bs, synth = c
    a = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    w = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    qa, sa, qw, sw = fp8bs.fp8_quant_linear(a, w)
    del a, w
    qc = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    scq = torch.empty(N // 128, M, dtype=torch.float32, device="cuda")
    cb = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    qc2 = torch.empty(M, N, dtype=torch.uint8, device="cuda")
    sc2 = torch.empty(N // 128, M, dtype=torch.float32, device="cuda")
    tm = Timer(torch)
    for i in range(iters + 5):
        f = lambda: fp8bs.fp8_block_gemm_e4m3_out(qa, sa, qw, sw, qc=qc, sc=scq)
        (tm.run("gemm_q", f) if i >= 5 else f())
        f2 = lambda: (fp8bs.fp8_block_gemm(qa, sa, qw, sw, out=cb),
                      fp8bs.fp8_quant_act_1x128(cb, qc2, sc2))
        (tm.run("gemm_then_q", f2) if i >= 5 else f2())
    ms, ms2 = tm.med_ms("gemm_q"), tm.med_ms("gemm_then_q")
    return {"us": ms * 1e3, **_flops_rate(2.0 * M * N * K, ms),
            "unfused_bf16_gemm_then_act_quant_us": ms2 * 1e3}


def part_quant_pair_step(c, iters):
    """The dense step's operands (4096x7168 activation, 18432x7168 weight):
    both quantized in one launch, timed interleaved with two launches."""
    torch, fp8bs, synth = c
    a = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    w = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    qa, sa, qw, sw = fp8bs.fp8_quant_linear(a, w)
    tm = Timer(torch)
    for i in range(iters + 5):
        f = lambda: fp8bs.fp8_quant_linear(a, w, qa, sa, qw, sw)
        (tm.run("q_pair", f) if i >= 5 else f())
        f2 = lambda: (fp8bs.fp8_quant_act_1x128(a, qa, sa), fp8bs.fp8_quant_w_128x128(w, qw, sw))
        (tm.run("q_two", f2) if i >= 5 else f2())
    ms, ms2 = tm.med_ms("q_pair"), tm.med_ms("q_two")
    byt = M * K * 3.03125 + N * K * (3.0 + 4.0 / 16384)
    return {"us": ms * 1e3, **_rate(byt, ms), "two_launches_us": ms2 * 1e3}


def part_moe(c, iters):
    """Grouped MoE: 4096 tokens, top-8 of 32 experts; gate/up N=4096 K=7168,
    down N=7168 K=2048; step = quantize the A's and all expert weights, then
    the two grouped GEMMs."""
    import numpy as np
    torch, fp8bs, synth = c
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
    tm = Timer(torch)

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
    for i in range(max(iters // 3, 5)):
        moe_step(True)
    f1 = 2.0 * Mt * 4096 * 7168
    f2 = 2.0 * Mt * 7168 * 2048
    g1, g2 = tm.med_ms("moe_g1"), tm.med_ms("moe_g2")
    tot = g1 + g2 + tm.med_ms("moe_qa") + tm.med_ms("moe_qw")

    def attainable_ms(N_, K_):
        """Per-expert roofline: sum over the experts of max(flops / P, bytes / BW),
        bytes = the expert's weight codes and block scales, its A rows with their
        scales, and its bf16 output rows (an empty expert reads nothing)."""
        t = 0.0
        for g in range(G):
            m = int(offsets[g + 1] - offsets[g])
            if m == 0:
                continue
            fl = 2.0 * m * N_ * K_
            by = N_ * K_ + (N_ // 128) * (K_ // 128) * 4 + m * K_ * (1 + 4 / 128) + m * N_ * 2
            t += max(fl / (PEAK_FP8_TFLOPS * 1e12), by / (PEAK_HBM_GBPS * 1e9))
        return t * 1e3

    att = attainable_ms(4096, 7168) + attainable_ms(7168, 2048)
    return {"M_total": Mt, "experts_empty": int((offsets[1:] == offsets[:-1]).sum()),
            "per_expert_attainable_us": att * 1e3,
            "gemms_frac_of_per_expert_attainable": att / (g1 + g2),
            "gate_up_us": g1 * 1e3, "gate_up_TFLOPs": f1 / g1 / 1e9,
            "down_us": g2 * 1e3, "down_TFLOPs": f2 / g2 / 1e9,
            "gemms_TFLOPs": (f1 + f2) / (g1 + g2) / 1e9,
            "gemms_frac_mfma": (f1 + f2) / (g1 + g2) / 1e9 / PEAK_FP8_TFLOPS,
            "step_with_quant_us": tot * 1e3, "step_TFLOPs": (f1 + f2) / tot / 1e9}


def part_moe_backward(c, iters):
    """MoE backward of the gate/up layer (same routing): data gradient
    dX = dY . W_g (grouped GEMM over per-expert transposed weights) and
    weight gradients dW_g = dY_g^T . X_g (one launch over the experts'
    128-padded token ranges)."""
    import numpy as np
    torch, fp8bs, synth = c
    G, T = 32, 4096
    order, offsets = synth.routing(T, G, 8, case=synth.MOE.case_id)
    Mt = int(offsets[-1])
    off_d = torch.from_numpy(offsets).cuda()
    tokens = synth.act(T, 7168, case=synth.MOE.case_id, tensor=0, device="cuda")
    a1 = tokens[torch.from_numpy(order).cuda()]
    del tokens
    w1 = synth.expert_weights(G, 4096, 7168, case=synth.MOE.case_id, tensor=10, device="cuda")
    dy1 = synth.act(Mt, 4096, case=synth.MOE.case_id, tensor=2, device="cuda")
    qwt = torch.empty(G, 7168, 4096, dtype=torch.uint8, device="cuda")
    swt = torch.empty(G, 56, 32, dtype=torch.float32, device="cuda")
    for g in range(G):
        _, _, qt, st = fp8bs.fp8_quant_w_128x128_t(w1[g])
        qwt[g].copy_(qt)
        swt[g].copy_(st)
    del w1
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
    tm = Timer(torch)

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
    for i in range(max(iters // 3, 5)):
        moe_bwd(True)
    fdx = 2.0 * Mt * 4096 * 7168
    fdw = 2.0 * Tp * 4096 * 7168  # padded tokens included (zero rows)
    tdx, tdw, tq = tm.med_ms("mb_dx"), tm.med_ms("mb_dw"), tm.med_ms("mb_q")
    return {"tokens_padded": Tp,
            "dgrad_us": tdx * 1e3, "dgrad_TFLOPs": fdx / tdx / 1e9,
            "wgrad_us": tdw * 1e3, "wgrad_TFLOPs": fdw / tdw / 1e9,
            "wgrad_useful_TFLOPs": fdx / tdw / 1e9,
            "wgrad_bf16_out_us": tm.med_ms("mb_dw16") * 1e3,
            "wgrad_bf16_out_TFLOPs": fdw / tm.med_ms("mb_dw16") / 1e9,
            "quantizers_us": tq * 1e3}


def part_backward(c, iters):
    """Backward pass of the dense layer (tokens 4096, N=18432, K=7168):
    quantizers with transposed outputs, data gradient dX = dY . W
    (contraction 18432) and weight gradient dW = dY^T . X (contraction
    4096)."""
    torch, fp8bs, synth = c
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
    tm = Timer(torch)

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
    return {"weight_quant_with_transpose_us": t["b_qw"] * 1e3,
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


def part_tiny(c, iters):
    """The tiny workload: quantize A 128x512 and W 256x512, GEMM with fp32
    output (launch-latency bound).  Timed as the step runs it (both quantizers
    in one launch, then the GEMM, into preallocated buffers), and as three
    separate calls that allocate their outputs."""
    torch, fp8bs, synth = c
    a, w = synth.tiny_inputs(device="cuda")
    M, K, N = a.shape[0], a.shape[1], w.shape[0]
    out = torch.empty(M, N, dtype=torch.float32, device="cuda")
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(K // 128, M, dtype=torch.float32, device="cuda")
    qw = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")

    def step(i):
        fp8bs.fp8_quant_linear(a, w, qa, sa, qw, sw)
        fp8bs.fp8_block_gemm(qa, sa, qw, sw, out=out)

    def three_calls(i):
        qa2, sa2 = fp8bs.fp8_quant_act_1x128(a)
        qw2, sw2 = fp8bs.fp8_quant_w_128x128(w)
        fp8bs.fp8_block_gemm(qa2, sa2, qw2, sw2, out=out)

    med, p10, p90 = _timeit(torch, step, iters)
    med3, _, _ = _timeit(torch, three_calls, iters)
    return {"us": med * 1e3, "p10_us": p10 * 1e3, "p90_us": p90 * 1e3,
            "three_allocating_calls_us": med3 * 1e3,
            "note": "two launches (both quantizers in one, then the GEMM) into preallocated "
                    "buffers; latency bound"}


def part_ablation(c, iters):
    """Online against delayed scaling on drifting activations (quality)."""
    from fp8_block_scaled_05_amd import ablation
    return ablation.run(steps=24, timing_iters=10)


PARTS = {
    "dense_gemm": part_dense_gemm,
    "e4m3_out": part_e4m3_out,
    "quant_pair_step": part_quant_pair_step,
    "act_quant": part_act_quant,
    "hbm_copy": part_hbm_copy,
    "weight_quant": part_weight_quant,
    "quant_pair": part_quant_pair,
    "skinny16": part_skinny16,
    "skinny64": part_skinny64,
    "moe": part_moe,
    "moe_backward": part_moe_backward,
    "backward": part_backward,
    "tiny": part_tiny,
    "ablation": part_ablation,
}

# keys of the parts in the bench line (named for their workloads)
PART_KEYS = {
    "e4m3_out": "dense_gemm_e4m3_out_M4096_N18432_K7168",
    "quant_pair_step": "quant_pair_one_launch_4096x7168_and_18432x7168",
    "act_quant": "act_quant_8192x7168",
    "hbm_copy": "hbm_copy_reference_177995776_bytes",
    "weight_quant": "weight_quant_18432x7168",
    "quant_pair": "quant_pair_8192x7168_and_18432x7168",
    "skinny16": "skinny_bf16_act_M16_N18432_K7168",
    "skinny64": "skinny_bf16_act_M64_N18432_K7168",
    "moe": "moe_grouped_E32_top8_T4096",
    "moe_backward": "moe_backward_gate_up_E32_top8_T4096",
    "backward": "backward_dense_M4096_N18432_K7168",
    "tiny": "tiny_M128_N256_K512",
    "ablation": "online_vs_delayed_scaling_M4096_K7168",
}


def _parts(ctx, iters=30):
    torch = ctx[0]
    out = {}
    for name, key in PART_KEYS.items():
        out[key] = PARTS[name](ctx, iters)
        torch.cuda.empty_cache()
    return out


def _rounded(v):
    if isinstance(v, dict):
        return {k: _rounded(x) for k, x in v.items()}
    if isinstance(v, float):
        return float(f"{v:.5g}")
    return v


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _cpu_baseline():
    """The oracle, as it stands, on the machine's host cores: the quantizer
    workload's two tensors in full (GB/s), the tiny workload in full, and
    the dense GEMM on 1024 of its 4096 rows (the metric's TFLOP/s; N and K
    full), about 25 s in all."""
    import numpy as np

    import oracle
    from fp8_block_scaled_05_amd import synth

    res = {}
    # tiny workload in full
    a, w = synth.tiny_inputs()
    t0 = time.perf_counter()
    qa, sa = oracle.quant_act_1x128(synth.bf16_bits(a))
    qw, sw = oracle.quant_w_128x128(synth.bf16_bits(w))
    oracle.block_gemm(qa, sa, qw, sw)
    res["tiny_full_s"] = time.perf_counter() - t0
    # quantizers on the full 8192x7168 activation and 18432x7168 weight
    x = synth.bf16_bits(synth.act(8192, K, case=synth.QUANT.case_id, tensor=0))
    t0 = time.perf_counter()
    oracle.quant_act_1x128(x)
    dt_a = time.perf_counter() - t0
    res["act_quant_8192x7168_GBps"] = 8192 * K * 3.03125 / dt_a / 1e9
    del x
    wb = synth.bf16_bits(synth.weight(N, K, case=synth.QUANT.case_id, tensor=10))
    t0 = time.perf_counter()
    qw, sw = oracle.quant_w_128x128(wb)
    dt_w = time.perf_counter() - t0
    res["weight_quant_18432x7168_GBps"] = N * K * (3.0 + 4.0 / 16384) / dt_w / 1e9
    del wb
    # dense GEMM on a row sample, float64 per-group sums
    Ms = 1024
    qa, sa = oracle.quant_act_1x128(
        synth.bf16_bits(synth.act(Ms, K, case=synth.DENSE.case_id, tensor=50)))
    t0 = time.perf_counter()
    oracle.block_gemm(qa, sa, qw, sw)
    dt_g = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    return {"value": 2.0 * Ms * N * K / dt_g / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"block GEMM (float64 per-group sums) on M={Ms} of the dense workload's "
                      f"4096 rows, N={N}, K={K}: {dt_g:.2f} s; also the act quantizer on the full "
                      f"8192x7168 ({dt_a:.2f} s) and the weight quantizer on the full 18432x7168 "
                      f"({dt_w:.2f} s), and the tiny workload in full",
            "cpu_model": _cpu_model(), "blas_threads": blas,
            "quantizers_and_tiny": _rounded(res)}


def _only(args):
    import torch

    from fp8_block_scaled_05_amd import fp8bs, synth
    if args.only not in PARTS:
        print(f"unknown part {args.only}; parts: {', '.join(PARTS)}", file=sys.stderr)
        sys.exit(2)
    res = PARTS[args.only]((torch, fp8bs, synth), args.iters)
    print(json.dumps({"part": args.only, "iters": args.iters, **_rounded(res)}), flush=True)


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)
    if args.only:
        _only(args)
        return

    import torch

    from fp8_block_scaled_05_amd import fp8bs, synth

    a = synth.act(M, K, case=synth.DENSE.case_id, tensor=0, device="cuda")
    w = synth.weight(N, K, case=synth.DENSE.case_id, tensor=1, device="cuda")
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(K // 128, M, dtype=torch.float32, device="cuda")
    qw = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sw = torch.empty(N // 128, K // 128, dtype=torch.float32, device="cuda")
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tm = Timer(torch)

    def step(timed):
        run = tm.run if timed else (lambda n, f: f())
        run("quant", lambda: fp8bs.fp8_quant_linear(a, w, qa, sa, qw, sw))
        run("gemm", lambda: fp8bs.fp8_block_gemm(qa, sa, qw, sw, out=c))

    clock = ClockStamps(torch)
    smi_before = _smi_snapshot()
    # settle the engine clock, then the W warm-up steps
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < CLOCK_SETTLE_S:
        for _ in range(20):
            step(False)
        settle_steps += 20
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(False)
    # the clock stamps sit just outside the timed region (the idle gaps
    # between them and the steps are a few microseconds of ~55 ms)
    clock.stamp(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clock.stamp(1)
    xcd_mhz = clock.mhz()
    smi_after = _smi_snapshot()
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
    clock_mhz = sum(xcd_mhz.values()) / len(xcd_mhz) if xcd_mhz else None

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
        "clock": {"engine_mhz_timed_mean_over_xcds": round(clock_mhz, 1) if clock_mhz else None,
                  "engine_mhz_per_xcd": ({str(k): round(v, 1) for k, v in xcd_mhz.items()}
                                         if xcd_mhz else None),
                  "source": ("cycle and wall-clock stamps around the timed steps "
                             "(tests/native/clock_probe.hip)") if xcd_mhz else None,
                  "settle_s": CLOCK_SETTLE_S, "settle_steps": settle_steps,
                  "peak_at_held_clock_TFLOPs": (round(PEAK_FP8_TFLOPS * clock_mhz / 2400.0, 1)
                                                if clock_mhz else None),
                  "frac_of_peak_at_held_clock": (round(gemm_tflops / (PEAK_FP8_TFLOPS * clock_mhz
                                                                       / 2400.0), 4)
                                                 if clock_mhz else None),
                  "smi_before_settle": smi_before, "smi_after_timed_steps": smi_after},
        "breakdown_us": {"quant_act_and_weight": round(q_ms * 1e3, 2),
                         "gemm": round(g_ms * 1e3, 2)},
        "quant_in_step": {"GBps": round(quant_bytes / q_ms / 1e6, 1),
                          "frac_hbm": round(quant_bytes / q_ms / 1e6 / PEAK_HBM_GBPS, 4)},
    }
    del a, w, c
    torch.cuda.empty_cache()
    if not args.no_parts:
        line["parts"] = _rounded(_parts((torch, fp8bs, synth)))
    line["cpu_baseline"] = None if args.no_cpu_baseline else _cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
