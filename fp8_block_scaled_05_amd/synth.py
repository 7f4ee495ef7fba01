"""Seeded synthetic inputs for the block-scaled FP8 path.

This module only draws random tensors; it holds none of the method's
arithmetic (no scaling, no FP8 encoding, no GEMM), so both the GPU path and
the CPU oracle can take their inputs from it.

Recipes (all values are drawn in float32 and cast to bfloat16 with
round-to-nearest-even at the end):

* ``act``: activations, N(0, 1) per element, each row multiplied by one
  LogNormal(0, 1) factor, then ``round(1e-3 * numel)`` distinct positions
  (uniform, without replacement) multiplied by the outlier factor (100 by
  default, 50 for the tiny case, which has no per-row factor).
* ``weight``: N(0, 0.02) per element (0.02 is the standard deviation).
* ``routing``: one global expert distribution p ~ Dirichlet(0.5 * 1_G); each
  token draws ``top_k`` distinct experts with probability proportional to p,
  without replacement.  Rows are then grouped by expert in token order.

The generator is ``torch.Generator`` seeded from (base seed, case id, tensor
id); tensors are generated on the requested device (CPU for sizes the oracle
handles in full, the GPU for full-size cases, whose sampled rows are copied to
the host for the oracle).  Routing uses NumPy's PCG64 on the host.
"""

from dataclasses import dataclass

import numpy as np
import torch

BASE_SEED = 0


def seed_for(case: int, tensor: int, base: int = BASE_SEED) -> int:
    return (base * 1_000_003 + case * 1_009 + tensor) & 0x7FFF_FFFF_FFFF


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def act(M, K, *, case, tensor=0, device="cpu", row_lognormal=True,
        outlier_frac=1e-3, outlier_mult=100.0):
    """bf16 [M][K] activation tensor (see module docstring)."""
    g = _gen(device, seed_for(case, tensor))
    x = torch.randn(M, K, generator=g, device=device, dtype=torch.float32)
    if row_lognormal and M:
        x *= torch.exp(torch.randn(M, 1, generator=g, device=device, dtype=torch.float32))
    n_out = int(round(outlier_frac * M * K))
    if n_out:
        idx = torch.randperm(M * K, generator=g, device=device)[:n_out]
        x.view(-1)[idx] *= outlier_mult
    return x.to(torch.bfloat16)


def drifting_act(M, K, step, *, case, growth=1.05, device="cpu"):
    """Activation tensor of training step ``step`` for the online vs delayed
    scaling comparison: a fresh draw of ``act`` per step (outliers move to
    new positions) times ``growth ** step`` (the distribution drifts)."""
    x = act(M, K, case=case, tensor=1000 + step, device=device).float()
    return (x * float(growth) ** step).to(torch.bfloat16)


def weight(N, K, *, case, tensor=1, device="cpu", std=0.02):
    """bf16 [N][K] weight tensor, N(0, std)."""
    g = _gen(device, seed_for(case, tensor))
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
    return (w * std).to(torch.bfloat16)


def expert_weights(G, N, K, *, case, tensor=10, device="cpu", std=0.02):
    """bf16 [G][N][K]: one N(0, std) weight per expert."""
    out = torch.empty(G, N, K, dtype=torch.bfloat16, device=device)
    for gi in range(G):
        out[gi] = weight(N, K, case=case, tensor=tensor + gi, device=device, std=std)
    return out


def routing(tokens, experts, top_k, *, case, tensor=5, alpha=0.5):
    """Token->expert assignment.

    Returns ``(order, offsets)``: ``order`` int64 [tokens*top_k] lists the
    token of each grouped row (rows of expert 0 first, each expert's tokens in
    token order); ``offsets`` int32 [experts+1] are the group boundaries.
    """
    rng = np.random.Generator(np.random.PCG64(seed_for(case, tensor)))
    p = rng.dirichlet(np.full(experts, alpha))
    choice = np.empty((tokens, top_k), dtype=np.int64)
    for t in range(tokens):
        choice[t] = rng.choice(experts, size=top_k, replace=False, p=p)
    counts = np.bincount(choice.ravel(), minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.empty(tokens * top_k, dtype=np.int64)
    fill = offsets[:-1].astype(np.int64).copy()
    for t in range(tokens):
        for e in choice[t]:
            order[fill[e]] = t
            fill[e] += 1
    return order, offsets


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bfloat16 tensor (copies from the device if
    needed)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


# ----------------------------------------------------------------------------
# Named workloads (shapes from the tiny, quantizer, dense, MoE and skinny
# cases).  ``case`` ids keep the seeds of different workloads apart.


@dataclass(frozen=True)
class Case:
    name: str
    case_id: int


TINY = Case("tiny_gemm_M128_N256_K512", 1)
QUANT = Case("quant_act_M8192_K7168_w_N18432_K7168", 2)
DENSE = Case("dense_gemm_M4096_N18432_K7168", 3)
MOE = Case("moe_grouped_E32_top8_T4096", 4)
SKINNY = Case("skinny_fused_M16_M64_N18432_K7168", 5)


def tiny_inputs(device="cpu"):
    """Tiny case: A 128x512 N(0,1) with 0.1% outliers x50; W 256x512."""
    a = act(128, 512, case=TINY.case_id, tensor=0, device=device,
            row_lognormal=False, outlier_mult=50.0)
    w = weight(256, 512, case=TINY.case_id, tensor=1, device=device)
    return a, w
