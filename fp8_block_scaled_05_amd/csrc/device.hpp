// Device-side numerics shared by the gfx950 kernels of libfp8bs.
//
// Scale rule of the online quantization (pages: "How online quantization in
// DeepSeek-V3 differs from delayed quantization", item 1; "How the unified
// E4M3 format adds to DeepSeek-V3's efficiency", section "Dynamic scaling
// and online quantization"): a group's largest magnitude is mapped to the top
// of the E4M3 range.  Readings fixed here and in the C header: the scale is
// s = RN32(a/448) with a = max(amax, 2^-64), values are multiplied by
// r = RN32(448/a) and converted with round-to-nearest-even, saturating at 448.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Compile-time loop: f(std::integral_constant<int, I>{}) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

constexpr float kE4M3Max = 448.0f;
constexpr float kScaleFloor = 0x1p-64f;

// Widen the two bf16 values packed in a dword (exact).
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

// DPP lane permutation helpers (within a row of 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over the 16 lanes of a DPP row; every lane receives it.  The steps
// swap neighbours (quad_perm 1,0,3,2), pairs (quad_perm 2,3,0,1), quads
// (row_half_mirror) and halves (row_mirror).  Max is exact and
// order-independent, so the result equals a sequential maximum.
__device__ __forceinline__ float max_row16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// Maximum over a whole wave64; every lane receives it.
__device__ __forceinline__ float max_wave64(float v) {
  v = max_row16(v);
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

// Scale and reciprocal of a group (IEEE float32 divisions).
__device__ __forceinline__ void group_scale(float amax, float& s, float& r) {
  const float a = fmaxf(amax, kScaleFloor);
  s = __fdiv_rn(a, kE4M3Max);
  r = __fdiv_rn(kE4M3Max, a);
}

// Two float32 values -> two E4M3 codes (RNE, saturating) into the low
// (HI=false) or high (HI=true) half of `old`.  Inputs are clamped to +-448
// first; the gfx950 convert rounds to nearest even into OCP E4M3.
template <bool HI>
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -kE4M3Max, kE4M3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4M3Max, kE4M3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

// Quantize 8 bf16 values (one u32x4) with reciprocal r -> 8 codes (u32x2).
__device__ __forceinline__ u32x2 quant8(const u32x4 v, float r) {
  uint32_t lo = cvt2_e4m3<false>(bf16_lo(v.x) * r, bf16_hi(v.x) * r, 0u);
  lo = cvt2_e4m3<true>(bf16_lo(v.y) * r, bf16_hi(v.y) * r, lo);
  uint32_t hi = cvt2_e4m3<false>(bf16_lo(v.z) * r, bf16_hi(v.z) * r, 0u);
  hi = cvt2_e4m3<true>(bf16_lo(v.w) * r, bf16_hi(v.w) * r, hi);
  return u32x2{lo, hi};
}

// Largest magnitude of the 8 bf16 values in a u32x4, as float32.
__device__ __forceinline__ float absmax8(const u32x4 v, float m) {
  m = fmaxf(m, fabsf(bf16_lo(v.x)));
  m = fmaxf(m, fabsf(bf16_hi(v.x)));
  m = fmaxf(m, fabsf(bf16_lo(v.y)));
  m = fmaxf(m, fabsf(bf16_hi(v.y)));
  m = fmaxf(m, fabsf(bf16_lo(v.z)));
  m = fmaxf(m, fabsf(bf16_hi(v.z)));
  m = fmaxf(m, fabsf(bf16_lo(v.w)));
  m = fmaxf(m, fabsf(bf16_hi(v.w)));
  return m;
}

// float32 -> bf16 bits, round to nearest even: gfx950's V_CVT_PK_BF16_F32
// (one instruction per pair of values), which the compiler selects for a
// float -> __bf16 conversion on this target.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// (lo, hi) -> one dword: lo in bits 15:0, hi in bits 31:16
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

}  // namespace fp8bs
