"""The C ABI from plain C: include/fp8bs.h compiles as C99 (and as C++17) with
warnings as errors, a C program links libfp8bs.so and gets the documented statuses from
calls that validation rejects before any HIP call (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_block_scaled_05_amd")

PROGRAM = r"""
#include <stdio.h>
#include "fp8bs.h"

int main(void) {
  uint16_t x[128] = {0};
  uint8_t q[128] = {0};
  float s[1] = {0.0f};
  /* K not a multiple of 128 */
  int a = fp8_quant_act_1x128(x, 1, 100, 128, q, 128, s, 1, NULL);
  /* NULL output pointer */
  int b = fp8_quant_w_128x128(x, 1, 128, 128, NULL, 128, s, NULL);
  /* nothing to do */
  int c = fp8_block_gemm(FP8BS_A_E4M3, NULL, 128, NULL, 0, NULL, 128, NULL, NULL, 1,
                         FP8BS_OUT_BF16, 0, 1, 128, NULL, 0, NULL);
  /* unknown output kind */
  int d = fp8_block_gemm(FP8BS_A_E4M3, q, 128, s, 1, q, 128, s, q, 1, 9, 1, 1, 128, NULL, 0,
                         NULL);
  printf("%d %d %d %d %s\n", a, b, c, d, fp8bs_status_string(a));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_plain_c_and_links(tmp_path):
    lib = os.path.join(PKG, "libfp8bs.so")
    if not os.path.exists(lib):
        pytest.skip("libfp8bs.so is not built")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", PKG, "-lfp8bs", f"-Wl,-rpath,{PKG}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    if shutil.which("g++") is not None:  # the same program as C++: extern "C" linkage
        cpp = tmp_path / "abi.cpp"
        cpp.write_text(PROGRAM)
        subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror",
                        "-I", os.path.join(ROOT, "include"), str(cpp), "-o", str(exe) + "xx",
                        "-L", PKG, "-lfp8bs", f"-Wl,-rpath,{PKG}"], check=True)
        out_cpp = subprocess.run([str(exe) + "xx"], check=True, capture_output=True,
                                 text=True).stdout.split()
        assert out_cpp == out
    import fp8_block_scaled_05_amd.fp8bs as fp8bs
    assert [int(v) for v in out[:4]] == [fp8bs.ERR_SHAPE, fp8bs.ERR_NULL, fp8bs.OK,
                                         fp8bs.ERR_DTYPE]
    assert " ".join(out[4:]) == fp8bs.lib.fp8bs_status_string(fp8bs.ERR_SHAPE).decode()
