// Online E4M3 quantizers for gfx950: one scale per 1x128 activation tile and
// per 128x128 weight block, computed from the group's current values on every
// call (pages: "How online quantization in DeepSeek-V3 differs from delayed
// quantization", items 1-3; "How the unified E4M3 format adds to
// DeepSeek-V3's efficiency", sections "Fine-grained quantization strategy"
// and "Dynamic scaling and online quantization").
//
// Both kernels are HBM-bound streams (2 bytes in, 1 byte + a scale out per
// element).  Each 16-lane DPP row owns one 256-byte row segment of a group:
// 16-byte loads, a DPP max across the row, the scale, then 8-byte code stores.

#include "device.hpp"
#include "internal.hpp"

namespace fp8bs {

namespace {

constexpr int kActRowsPerWG = 64;   // rows of one 1x128 column of tiles per workgroup
constexpr int kActIters = kActRowsPerWG / 16;

// grid: one workgroup per (64-row band, K group), K group fastest so that
// consecutive workgroups walk along the same rows.
__global__ __launch_bounds__(256) void quant_act_1x128_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t KB, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s, int64_t lds) {
  const int64_t bid = blockIdx.x;
  const int64_t kb = bid % KB;
  const int64_t m0 = (bid / KB) * kActRowsPerWG;
  const int lane = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;

  u32x4 v[kActIters];
#pragma unroll
  for (int i = 0; i < kActIters; ++i) {
    int64_t m = m0 + grp + 16 * i;
    m = m < M ? m : M - 1;
    v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(x + m * ldx + kb * 128) + lane);
  }
#pragma unroll
  for (int i = 0; i < kActIters; ++i) {
    const int64_t m = m0 + grp + 16 * i;
    const float amax = max_row16(absmax8(v[i], 0.0f));
    float sc, r;
    group_scale(amax, sc, r);
    const u32x2 codes = quant8(v[i], r);
    if (m < M) {
      __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + m * ldq + kb * 128) + lane);
      if (lane == 0) s[kb * lds + m] = sc;
    }
  }
}

// grid: one workgroup per 128x128 block, K group fastest.  Each thread holds
// 8 row segments of 8 values (the block stays in registers: one HBM pass).
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t KB, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ s) {
  __shared__ float wave_max[4];
  const int64_t bid = blockIdx.x;
  const int64_t kb = bid % KB;
  const int64_t nb = bid / KB;
  const int lane = threadIdx.x & 15;
  const int r0 = threadIdx.x >> 4;

  u32x4 v[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = nb * 128 + r0 + 16 * i;
    const int64_t nc = n < N ? n : N - 1;
    v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(w + nc * ldw + kb * 128) + lane);
    // rows past N belong to no block: they must not raise the maximum
    if (n >= N) v[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) m = absmax8(v[i], m);
  m = max_wave64(m);
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  float sc, r;
  group_scale(amax, sc, r);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = nb * 128 + r0 + 16 * i;
    if (n < N) {
      const u32x2 codes = quant8(v[i], r);
      __builtin_nontemporal_store(codes, reinterpret_cast<u32x2*>(q + n * ldq + kb * 128) + lane);
    }
  }
  if (threadIdx.x == 0) s[nb * KB + kb] = sc;
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            hipStream_t stream) {
  const int64_t KB = K / 128;
  const int64_t MB = (M + kActRowsPerWG - 1) / kActRowsPerWG;
  const int64_t blocks = MB * KB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_act_1x128_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     x, M, KB, ldx, q, ldq, s, lds);
  return hipGetLastError();
}

hipError_t launch_quant_w(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                          uint8_t* q, int64_t ldq, float* s, hipStream_t stream) {
  const int64_t KB = K / 128;
  const int64_t NB = (N + 127) / 128;
  const int64_t blocks = NB * KB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(quant_w_128x128_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     w, N, KB, ldw, q, ldq, s);
  return hipGetLastError();
}

}  // namespace fp8bs
