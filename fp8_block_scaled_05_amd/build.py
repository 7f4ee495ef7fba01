"""Build libfp8bs.so (hand-written HIP for gfx950) in-tree with hipcc, and
the test-only kernel libraries under tests/native.

Usage: ``python -m fp8_block_scaled_05_amd.build`` (also called by
``__graft_entry__.build()``).  Always recompiles.
"""

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp8bs.so")
# test and measurement helpers (never part of libfp8bs): tests/native/*.hip,
# each built into its own library next to its source, with the package's
# device headers (the convert sweep of the GPU tests, bench.py's clock stamps)
TEST_NATIVE = os.path.join(ROOT, "tests", "native")
ARCH = "gfx950"

# Packed-FP32 VALU instructions are disabled for all device code; the
# compiler otherwise forms them from ordinary float code.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source additions.  The few-row kernels run one wave per SIMD, where the
# compiler would put MFMA results in accumulation registers and copy each
# one out before its FP32 promotion; this option keeps them in VGPRs.
EXTRA_FLAGS = {"gemm_few_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; it is needed to build libfp8bs.so")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under " + CSRC)

    def compile_one(src):
        obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
        extra = EXTRA_FLAGS.get(os.path.basename(src), [])
        cmd = [hipcc, *DEVICE_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    for src in sorted(glob.glob(os.path.join(TEST_NATIVE, "*.hip"))):
        out = os.path.join(TEST_NATIVE, "lib" + os.path.basename(src)[:-4] + ".so")
        cmd = [hipcc, *DEVICE_FLAGS, "-I", CSRC, "-shared", src, "-o", out + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
