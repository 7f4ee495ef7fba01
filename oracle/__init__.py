"""CPU oracle for block-scaled FP8 (online 1x128 / 128x128 quantization to E4M3
and the FP32-promoted block GEMM).

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
NumPy restatement of what the GPU path computes.  It exists so that the HIP
kernels can be checked against something that shares none of their code.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (``fp8_block_scaled_05_amd``)
never does, and must fail loudly rather than fall back to it.

Sources (cited by page title and section; the pages are knowledge-base answers
about DeepSeek-V3 on codingmall.com):

* "How online quantization in DeepSeek-V3 differs from delayed quantization",
  items 1-3: a scale is computed on the fly from the current 1x128 activation
  tile or 128x128 weight block, with no stored history of maxima.
* "How the unified E4M3 format adds to DeepSeek-V3's efficiency", sections
  "Fine-grained quantization strategy" and "Dynamic scaling and online
  quantization": E4M3 is the only FP8 format; activations are grouped per
  1x128 tile and weights per 128x128 block, and each group's scale spreads its
  values over the representable FP8 values.  Section "Enhanced numerical
  stability": partial sums are promoted to FP32 registers at fixed intervals
  of the accumulation.
* "Advantages of using FP8 for GEMM operations in DeepSeek-V3", items 4-8:
  the same grouping, FP32 promotion, universal E4M3, online scaling, and a
  GEMM library covering dense and MoE layers.

Where the pages leave a parameter open (E4M3 variant, scale formula, rounding,
saturation, the promotion interval, tiny tiles, layouts), the readings taken
are listed in the module docstrings below; every one of them is fixed the same
way on the GPU side.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(closed forms, a library decode, brute force on tiny inputs, invariants).
The only unpinned aspect is the GPU's own summation order inside one 128-K
block, which the GEMM tolerance covers.
"""

from .e4m3 import E4M3_MAX, decode, decode_table, encode  # noqa: F401
from .quant import (  # noqa: F401
    SCALE_FLOOR,
    quant_act_1x128,
    quant_rows_1x128,
    quant_w_128x128,
    tile_scale,
)
from .backward import (  # noqa: F401
    block_gemm_rowscaled,
    dgrad,
    kgrouped_gemm_rowscaled,
    quant_act_128x1_t,
    quant_w_128x128_t,
    wgrad,
)
from .delayed import quant_act_1x128_delayed  # noqa: F401
from .gemm import (  # noqa: F401
    block_gemm,
    block_gemm_e4m3_out,
    block_grouped_gemm,
    fused_act_gemm,
)
