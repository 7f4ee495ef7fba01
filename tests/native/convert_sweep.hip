// Test-only kernels (not part of libfp8bs, not declared in fp8bs.h):
// - a contiguous range of float32 bit patterns through the library's own
//   device convert (cvt2_e4m3 in device.hpp: clamp to +-448, then the gfx950
//   round-to-nearest-even convert to OCP E4M3), one code per input; the GPU
//   parity test compares the codes of every non-NaN float32 value with the
//   oracle's table-search encoder;
// - given float32 bit patterns through the library's bf16 output rounding
//   (bf16x2_rne and f32_to_bf16_rne in device.hpp: gfx950's
//   V_CVT_PK_BF16_F32), one bf16 pattern per input, which the test compares
//   with a CPU round-to-nearest-even conversion.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace {

// The convert without the clamp: the few-row GEMM's in-kernel activation
// quantizer skips the clamp, which changes nothing for finite inputs only if
// the hardware convert takes every |y| in [448, 464) to the code of 448.
__device__ __forceinline__ uint32_t cvt2_raw(float a, float b, uint32_t old, bool hi) {
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}

// codes[i] = E4M3(bits first + i) for i < n; 8 inputs per thread.  RAW: the
// bare hardware convert, else the library's clamped cvt2_e4m3.
template <bool RAW>
__global__ __launch_bounds__(256) void convert_range_kernel(uint32_t first, int64_t n,
                                                            uint8_t* __restrict__ codes) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= n) return;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    x[j] = i0 + j < n ? __uint_as_float(first + (uint32_t)(i0 + j)) : 0.0f;
  uint32_t lo, hi;
  if constexpr (RAW) {
    lo = cvt2_raw(x[2], x[3], cvt2_raw(x[0], x[1], 0u, false), true);
    hi = cvt2_raw(x[6], x[7], cvt2_raw(x[4], x[5], 0u, false), true);
  } else {
    lo = fp8bs::cvt2_e4m3<true>(x[2], x[3], fp8bs::cvt2_e4m3<false>(x[0], x[1], 0u));
    hi = fp8bs::cvt2_e4m3<true>(x[6], x[7], fp8bs::cvt2_e4m3<false>(x[4], x[5], 0u));
  }
  if (i0 + 8 <= n) {
    *reinterpret_cast<fp8bs::u32x2*>(codes + i0) = fp8bs::u32x2{lo, hi};
  } else {
    for (int j = 0; i0 + j < n; ++j)
      codes[i0 + j] = (uint8_t)((j < 4 ? lo : hi) >> (8 * (j & 3)));
  }
}

// out[i] = bf16(in[i]): even i through the paired convert (with in[i + 1]),
// the last element of an odd count through the single one.
__global__ __launch_bounds__(256) void bf16_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                   uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
  if (i >= n) return;
  if (i + 1 < n) {
    const uint32_t w = fp8bs::bf16x2_rne(__uint_as_float(in[i]), __uint_as_float(in[i + 1]));
    out[i] = (uint16_t)w;
    out[i + 1] = (uint16_t)(w >> 16);
  } else {
    out[i] = fp8bs::f32_to_bf16_rne(__uint_as_float(in[i]));
  }
}

}  // namespace

// Returns 0 on success, 2 for an empty or too large count, or the HIP error
// of the launch.
extern "C" int fp8bs_test_bf16_convert(const uint32_t* in, int64_t n, uint16_t* out,
                                       void* stream) {
  if (n <= 0 || n > (int64_t(1) << 34)) return 2;
  const int64_t blocks = (n + 511) / 512;
  void* args[] = {&in, &n, &out};
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(bf16_kernel), dim3((unsigned)blocks),
                              dim3(256), args, 0, static_cast<hipStream_t>(stream));
}

// raw != 0: the bare convert (no clamp).  Returns 0 on success, 2 for a
// range that is empty, wraps past 0xFFFFFFFF or is too large for one launch,
// 3 for a misaligned output, or the HIP error of the launch.
extern "C" int fp8bs_test_convert_range(uint32_t first, int64_t n, uint8_t* codes, int raw,
                                        void* stream) {
  if (n <= 0 || (uint64_t)first + (uint64_t)n - 1 > 0xFFFFFFFFull || n > (int64_t(1) << 34))
    return 2;
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0) return 3;
  const int64_t blocks = (n + 2047) / 2048;
  void* args[] = {&first, &n, &codes};
  const void* k = raw ? reinterpret_cast<const void*>(convert_range_kernel<true>)
                     : reinterpret_cast<const void*>(convert_range_kernel<false>);
  return (int)hipLaunchKernel(k,
                              dim3((unsigned)blocks), dim3(256), args, 0,
                              static_cast<hipStream_t>(stream));
}
