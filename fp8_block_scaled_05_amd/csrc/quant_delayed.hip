// Delayed (history-based) scaling of 1x128 activation tiles for gfx950: the
// baseline that online scaling is compared against (pages: "How online
// quantization in DeepSeek-V3 differs from delayed quantization", items 2-4:
// delayed quantization derives its scales from maxima of earlier iterations,
// kept in a stored history).
//
// The scale of step t comes from the largest magnitude over steps t-H..t-1,
// by the online scale rule; a group with an empty window (maximum 0) is
// scaled from its current maximum.  Two granularities:
//   per tile:   ring hist[H][KB][ldh], step u in slot u % H; the 16 lanes of
//               a tile's row read its H slots, 16 at a time, and reduce them
//               by DPP max; lane 0 then stores the current maximum in slot
//               t % H (the tile has one owner, so no race);
//   per tensor: ring hist[H + 2], step u in slot u % (H + 2); every workgroup
//               reads the H window slots, raises slot t % (H + 2) to its
//               maximum with an atomic max, and workgroup 0 clears slot
//               (t + 1) % (H + 2) for the next step (no slot is both read and
//               written).  The
//               atomics of all workgroups meet at one address, so a
//               workgroup first reads the slot and skips the atomic when its
//               maximum cannot raise it (the slot only grows during a step).
// Values that the stale scale pushes past the format saturate; clipped
// (|x r| > 464, where round-to-nearest would leave the format) and flushed
// (non-zero, zero code) values are counted with one atomic add per wave.

#include "device.hpp"
#include "internal.hpp"

namespace fp8bs {

namespace {

constexpr int kRows = 64;  // rows of one column of tiles per workgroup
constexpr int kIters = kRows / 16;

struct DelayArgs {
  const uint16_t* x;
  int64_t M, KB, ldx;
  uint8_t* q;
  int64_t ldq;
  float* s;
  int64_t lds;
  float* hist;
  int64_t ldh, H, step;
  uint32_t* stats;  // [clipped, flushed] or null
};

// 8 bf16 values scaled by r -> 8 codes, counting clipped and flushed values.
__device__ __forceinline__ u32x2 quant8_counted(const u32x4 v, float r, uint32_t& clipped,
                                                uint32_t& flushed) {
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = x[k] * r;
    clipped += fabsf(y[k]) > 464.0f ? 1u : 0u;
  }
  uint32_t lo = cvt2_e4m3<false>(y[0], y[1], 0u);
  lo = cvt2_e4m3<true>(y[2], y[3], lo);
  uint32_t hi = cvt2_e4m3<false>(y[4], y[5], 0u);
  hi = cvt2_e4m3<true>(y[6], y[7], hi);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t code = ((k < 4 ? lo : hi) >> (8 * (k & 3))) & 0x7Fu;
    flushed += (code == 0u && x[k] != 0.0f) ? 1u : 0u;
  }
  return u32x2{lo, hi};
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += (uint32_t)__shfl_xor((int)v, o, 64);
  return v;
}

// grid: one workgroup per (64-row band, K group), K group fastest.
template <bool TENSOR>
__global__ __launch_bounds__(256) void quant_act_delayed_kernel(DelayArgs a) {
  __shared__ float wave_max[4];
  const int64_t bid = blockIdx.x;
  const int64_t kb = bid % a.KB;
  const int64_t m0 = (bid / a.KB) * kRows;
  const int lane = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;

  u32x4 v[kIters];
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    int64_t m = m0 + grp + 16 * i;
    m = m < a.M ? m : a.M - 1;
    v[i] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(a.x + m * a.ldx + kb * 128) + lane);
  }
  const int64_t ring = TENSOR ? a.H + 2 : a.H;
  float win_tensor = 0.0f;
  if constexpr (TENSOR) {
    // the window's H slots, 64 at a time across the wave's lanes
    const int l64 = threadIdx.x & 63;
    for (int64_t h0 = 0; h0 < a.H; h0 += 64) {
      const int64_t d = h0 + l64;
      if (d < a.H) win_tensor = fmaxf(win_tensor, a.hist[((a.step - 1 - d) % ring + ring) % ring]);
    }
    win_tensor = max_wave64(win_tensor);
  }
  uint32_t clipped = 0, flushed = 0;
  float tmax = 0.0f;
#pragma unroll
  for (int i = 0; i < kIters; ++i) {
    const int64_t m = m0 + grp + 16 * i;
    const int64_t mc = m < a.M ? m : a.M - 1;
    const float cur = max_row16(absmax8(v[i], 0.0f));
    float win = win_tensor;
    if constexpr (!TENSOR) {
      for (int64_t h0 = 0; h0 < a.H; h0 += 16) {
        const int64_t h = h0 + lane;
        win = fmaxf(win, h < a.H ? a.hist[(h * a.KB + kb) * a.ldh + mc] : 0.0f);
      }
      win = max_row16(win);
    }
    float sc, r;
    group_scale(win > 0.0f ? win : cur, sc, r);
    uint32_t c = 0, f = 0;
    const u32x2 codes = quant8_counted(v[i], r, c, f);
    if (m < a.M) {
      clipped += c;
      flushed += f;
      tmax = fmaxf(tmax, cur);
      __builtin_nontemporal_store(codes,
                                  reinterpret_cast<u32x2*>(a.q + m * a.ldq + kb * 128) + lane);
      if (lane == 0) {
        a.s[kb * a.lds + m] = sc;
        if constexpr (!TENSOR) a.hist[((a.step % ring) * a.KB + kb) * a.ldh + m] = cur;
      }
    }
  }
  if constexpr (TENSOR) {
    tmax = max_wave64(tmax);
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = tmax;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float wmax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
      // non-negative floats order like their bit patterns
      unsigned int* const slot = reinterpret_cast<unsigned int*>(a.hist + a.step % ring);
      if (__float_as_uint(wmax) > __atomic_load_n(slot, __ATOMIC_RELAXED))
        atomicMax(slot, __float_as_uint(wmax));
      // one workgroup clears the next step's slot (the next call is ordered
      // after this one on its stream); a store from every workgroup to one
      // address would serialize them
      if (bid == 0) a.hist[(a.step + 1) % ring] = 0.0f;
    }
  }
  if (a.stats) {
    clipped = wave_sum_u32(clipped);
    flushed = wave_sum_u32(flushed);
    if ((threadIdx.x & 63) == 0) {
      if (clipped) atomicAdd(a.stats, clipped);
      if (flushed) atomicAdd(a.stats + 1, flushed);
    }
  }
}

}  // namespace

hipError_t launch_quant_act_delayed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                    uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                    bool per_tensor, float* hist, int64_t ldh, int64_t H,
                                    int64_t step, uint32_t* stats, hipStream_t stream) {
  DelayArgs a{x, M, K / 128, ldx, q, ldq, s, lds, hist, ldh, H, step, stats};
  const int64_t blocks = (M + kRows - 1) / kRows * a.KB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (per_tensor)
    return launch_kernel(quant_act_delayed_kernel<true>, dim3((unsigned)blocks), dim3(256),
                         stream, a);
  return launch_kernel(quant_act_delayed_kernel<false>, dim3((unsigned)blocks), dim3(256), stream,
                       a);
}

}  // namespace fp8bs
