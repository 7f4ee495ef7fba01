"""Block-scaled FP8 for AMD MI355X (gfx950).

Online 1x128 / 128x128 quantization to E4M3 and the FP32-promoted block GEMM
(dense, grouped, skinny with fused activation quantization), implemented as
hand-written HIP kernels behind the C ABI declared in ``include/fp8bs.h``.

``fp8_block_scaled_05_amd.fp8bs`` is the thin ctypes binding over that
library; importing it loads ``libfp8bs.so`` and raises if it is missing.
``fp8_block_scaled_05_amd.synth`` draws seeded synthetic inputs.
"""
