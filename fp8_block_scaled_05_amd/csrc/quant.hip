// Online E4M3 quantizers for gfx950: one scale per 1x128 activation tile and
// per 128x128 weight block, computed from the group's current values on every
// call (pages: "How online quantization in DeepSeek-V3 differs from delayed
// quantization", items 1-3; "How the unified E4M3 format adds to
// DeepSeek-V3's efficiency", sections "Fine-grained quantization strategy"
// and "Dynamic scaling and online quantization").
//
// All kernels here are HBM-bound streams (2 bytes in, 1 byte + a scale out
// per element).  Each 16-lane DPP row owns one 256-byte row segment of a
// group: 16-byte loads, a DPP max across the row, the scale, then 8-byte code
// stores.  Kernels: the 1x128 activation quantizer, the 128x128 weight
// quantizer (optionally also writing W^T), both in one launch for a linear
// layer's two operands, and the 128-token transposed activation quantizer of
// the weight gradient.

#include "device.hpp"
#include "internal.hpp"

namespace fp8bs {

namespace {

constexpr int kActRowsPerWG = 64;   // rows of one 1x128 column of tiles per workgroup
constexpr int kActIters = kActRowsPerWG / 16;

struct ActArgs {
  const uint16_t* x;
  int64_t M, KB, ldx;
  uint8_t* q;
  int64_t ldq;
  float* s;
  int64_t lds;
};

struct WArgs {
  const uint16_t* w;
  int64_t N, KB, ldw;
  uint8_t* q;
  int64_t ldq;
  float* s;
  uint8_t* qt;
  int64_t ldqt;
  float* st;
};

// Work item `bid` of the activation quantizer: one (64-row band, K group),
// K group fastest so that consecutive workgroups walk along the same rows.
__device__ __forceinline__ void act_band(const ActArgs& a, int64_t bid) {
  const uint16_t* __restrict__ x = a.x;
  uint8_t* __restrict__ q = a.q;
  float* __restrict__ s = a.s;
  const int64_t M = a.M, KB = a.KB, ldx = a.ldx, ldq = a.ldq, lds = a.lds;
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

__global__ __launch_bounds__(256) void quant_act_1x128_kernel(ActArgs a) {
  act_band(a, blockIdx.x);
}

// Transpose of an 8x8 byte block: row i is (lo[i], hi[i]) (bytes 0..3, 4..7);
// returns column c as (olo[c], ohi[c]) = bytes c of rows 0..3 and 4..7.
// v_perm_b32 picks each result byte from the 8 bytes {S0 (4..7), S1 (0..3)}.
__device__ __forceinline__ void transpose8x8(const uint32_t (&lo)[8], const uint32_t (&hi)[8],
                                             uint32_t (&olo)[8], uint32_t (&ohi)[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t (&src)[8] = c < 4 ? lo : hi;
    const uint32_t b = (uint32_t)(c & 3);
    const uint32_t pick = b | ((4u + b) << 8);  // byte b of S1, then byte b of S0
    const uint32_t r01 = __builtin_amdgcn_perm(src[1], src[0], pick);
    const uint32_t r23 = __builtin_amdgcn_perm(src[3], src[2], pick);
    const uint32_t r45 = __builtin_amdgcn_perm(src[5], src[4], pick);
    const uint32_t r67 = __builtin_amdgcn_perm(src[7], src[6], pick);
    olo[c] = __builtin_amdgcn_perm(r23, r01, 0x05040100u);
    ohi[c] = __builtin_amdgcn_perm(r67, r45, 0x05040100u);
  }
}

// grid: one workgroup per 128x128 block, K group fastest.  Each thread holds
// 8 row segments of 8 values (the block stays in registers: one HBM pass).
// TRANS: the codes are also written transposed (qt [K][ldqt], N contiguous)
// with the transposed scale grid st [K/128][N/128], the B operand of the
// data-gradient GEMM dX = dY . W.  The block's codes go through LDS; each
// thread then reads an 8x8 byte block, transposes it in registers and writes
// eight 8-byte row pieces of qt.
template <bool TRANS>
__device__ __forceinline__ void w_block(const WArgs& a, int64_t bid) {
  const uint16_t* __restrict__ w = a.w;
  uint8_t* __restrict__ q = a.q;
  float* __restrict__ s = a.s;
  uint8_t* __restrict__ qt = a.qt;
  float* __restrict__ st = a.st;
  const int64_t N = a.N, KB = a.KB, ldw = a.ldw, ldq = a.ldq, ldqt = a.ldqt;
  __shared__ float wave_max[4];
  constexpr int kPitch = 136;  // LDS row pitch of the staged codes (bytes)
  __shared__ __attribute__((aligned(16))) uint8_t tile[TRANS ? 128 * kPitch : 8];
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
    const u32x2 codes = quant8(v[i], r);
    // plain code stores (nontemporal ones measured 7% slower for this
    // kernel); the loads stay nontemporal
    if (n < N) *(reinterpret_cast<u32x2*>(q + n * ldq + kb * 128) + lane) = codes;
    if constexpr (TRANS)
      *reinterpret_cast<u32x2*>(tile + (r0 + 16 * i) * kPitch + lane * 8) = codes;
  }
  if (threadIdx.x == 0) s[nb * KB + kb] = sc;
  if constexpr (TRANS) {
    // N % 128 == 0 here: every row of the block is real
    __syncthreads();
    const int n0 = (threadIdx.x & 15) * 8, k0 = (threadIdx.x >> 4) * 8;
    uint32_t lo[8], hi[8], olo[8], ohi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x2 d = *reinterpret_cast<const u32x2*>(tile + (n0 + i) * kPitch + k0);
      lo[i] = d.x;
      hi[i] = d.y;
    }
    transpose8x8(lo, hi, olo, ohi);
    const int64_t NB = N / 128;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int64_t k = kb * 128 + k0 + c;
      __builtin_nontemporal_store(u32x2{olo[c], ohi[c]},
                                  reinterpret_cast<u32x2*>(qt + k * ldqt + nb * 128 + n0));
    }
    if (threadIdx.x == 0) st[kb * NB + nb] = sc;
  }
}

template <bool TRANS>
__global__ __launch_bounds__(256) void quant_w_128x128_kernel(WArgs a) {
  w_block<TRANS>(a, blockIdx.x);
}

// Both operands of a forward linear layer in one launch: workgroups
// [0, w_blocks) quantize the weight's 128x128 blocks, the rest the
// activation's 1x128 tiles.  The activation's short stream then fills the
// end of the weight stream instead of paying its own launch ramp and drain.
__global__ __launch_bounds__(256) void quant_linear_kernel(ActArgs a, WArgs w, int64_t w_blocks) {
  const int64_t bid = blockIdx.x;
  if (bid < w_blocks) {
    w_block<false>(w, bid);
  } else {
    act_band(a, bid - w_blocks);
  }
}

// Groups of 128 consecutive rows per column (the 1x128 tiles of x^T), the
// operands of the weight-gradient GEMM dW = dY^T . X, which contracts over
// the tokens.  One workgroup per 128x128 block (N block fastest); each
// thread holds 8 row pieces of 8 values.  Column maxima: over the thread's
// rows, across the 4 row groups of a wave by shuffles, across the 4 waves
// in LDS; one thread per column forms its scale and reciprocal.  The codes
// are staged in LDS and written transposed (qt [N][M]) in 8x8 byte blocks.
__global__ __launch_bounds__(256) void quant_act_128x1_t_kernel(
    const uint16_t* __restrict__ x, int64_t NB, int64_t ldx, uint8_t* __restrict__ qt,
    int64_t ldqt, float* __restrict__ st, int64_t ldst) {
  constexpr int kPitch = 136;
  __shared__ float colmax[4][128];
  __shared__ __attribute__((aligned(16))) float rcp[128];
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kPitch];
  const int64_t bid = blockIdx.x;
  const int64_t nb = bid % NB;
  const int64_t mb = bid / NB;
  const int lane = threadIdx.x & 15;
  const int r0 = threadIdx.x >> 4;

  u32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
               x + (mb * 128 + r0 + 16 * i) * ldx + nb * 128) + lane);
  float cm[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) cm[c] = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 d = v[i];
    cm[0] = fmaxf(cm[0], fabsf(bf16_lo(d.x)));
    cm[1] = fmaxf(cm[1], fabsf(bf16_hi(d.x)));
    cm[2] = fmaxf(cm[2], fabsf(bf16_lo(d.y)));
    cm[3] = fmaxf(cm[3], fabsf(bf16_hi(d.y)));
    cm[4] = fmaxf(cm[4], fabsf(bf16_lo(d.z)));
    cm[5] = fmaxf(cm[5], fabsf(bf16_hi(d.z)));
    cm[6] = fmaxf(cm[6], fabsf(bf16_lo(d.w)));
    cm[7] = fmaxf(cm[7], fabsf(bf16_hi(d.w)));
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    cm[c] = fmaxf(cm[c], __shfl_xor(cm[c], 16, 64));
    cm[c] = fmaxf(cm[c], __shfl_xor(cm[c], 32, 64));
  }
  if ((threadIdx.x & 63) < 16) {
#pragma unroll
    for (int c = 0; c < 8; ++c) colmax[threadIdx.x >> 6][lane * 8 + c] = cm[c];
  }
  __syncthreads();
  if (threadIdx.x < 128) {
    const int col = threadIdx.x;
    const float amax = fmaxf(fmaxf(colmax[0][col], colmax[1][col]),
                             fmaxf(colmax[2][col], colmax[3][col]));
    float sc, r;
    group_scale(amax, sc, r);
    rcp[col] = r;
    st[mb * ldst + nb * 128 + col] = sc;
  }
  __syncthreads();
  const float4 ra = *reinterpret_cast<const float4*>(rcp + lane * 8);
  const float4 rb = *reinterpret_cast<const float4*>(rcp + lane * 8 + 4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x4 d = v[i];
    uint32_t lo = cvt2_e4m3<false>(bf16_lo(d.x) * ra.x, bf16_hi(d.x) * ra.y, 0u);
    lo = cvt2_e4m3<true>(bf16_lo(d.y) * ra.z, bf16_hi(d.y) * ra.w, lo);
    uint32_t hi = cvt2_e4m3<false>(bf16_lo(d.z) * rb.x, bf16_hi(d.z) * rb.y, 0u);
    hi = cvt2_e4m3<true>(bf16_lo(d.w) * rb.z, bf16_hi(d.w) * rb.w, hi);
    *reinterpret_cast<u32x2*>(tile + (r0 + 16 * i) * kPitch + lane * 8) = u32x2{lo, hi};
  }
  __syncthreads();
  // 16 consecutive threads cover the 128 tokens of one output row (whole
  // 128-byte lines per store)
  const int m0 = (threadIdx.x & 15) * 8, c0 = (threadIdx.x >> 4) * 8;
  uint32_t lo[8], hi[8], olo[8], ohi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const u32x2 d = *reinterpret_cast<const u32x2*>(tile + (m0 + i) * kPitch + c0);
    lo[i] = d.x;
    hi[i] = d.y;
  }
  transpose8x8(lo, hi, olo, ohi);
  // plain stores here (nontemporal ones measured 16% slower for this
  // kernel, the other way round from the weight transpose above)
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int64_t n = nb * 128 + c0 + c;
    *reinterpret_cast<u32x2*>(qt + n * ldqt + mb * 128 + m0) = u32x2{olo[c], ohi[c]};
  }
}

}  // namespace

hipError_t launch_quant_act_128x1_t(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                                    uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                                    hipStream_t stream) {
  const int64_t NB = N / 128;
  const int64_t blocks = (M / 128) * NB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return launch_kernel(quant_act_128x1_t_kernel, dim3((unsigned)blocks), dim3(256), stream, x,
                       NB, ldx, qt, ldqt, st, ldst);
}

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            hipStream_t stream) {
  const int64_t KB = K / 128;
  const int64_t MB = (M + kActRowsPerWG - 1) / kActRowsPerWG;
  const int64_t blocks = MB * KB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return launch_kernel(quant_act_1x128_kernel, dim3((unsigned)blocks), dim3(256), stream,
                       ActArgs{x, M, KB, ldx, q, ldq, s, lds});
}

hipError_t launch_quant_w(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                          uint8_t* q, int64_t ldq, float* s, uint8_t* qt, int64_t ldqt,
                          float* st, hipStream_t stream) {
  const int64_t KB = K / 128;
  const int64_t NB = (N + 127) / 128;
  const int64_t blocks = NB * KB;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const WArgs a{w, N, KB, ldw, q, ldq, s, qt, ldqt, st};
  if (qt) return launch_kernel(quant_w_128x128_kernel<true>, dim3((unsigned)blocks), dim3(256),
                               stream, a);
  return launch_kernel(quant_w_128x128_kernel<false>, dim3((unsigned)blocks), dim3(256), stream,
                       a);
}

hipError_t launch_quant_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               const uint16_t* w, int64_t N, int64_t ldw, uint8_t* qw,
                               int64_t ldqw, float* sw, hipStream_t stream) {
  const int64_t KB = K / 128;
  const int64_t w_blocks = (N + 127) / 128 * KB;
  const int64_t a_blocks = (M + kActRowsPerWG - 1) / kActRowsPerWG * KB;
  const int64_t blocks = w_blocks + a_blocks;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return launch_kernel(quant_linear_kernel, dim3((unsigned)blocks), dim3(256), stream,
                       ActArgs{x, M, KB, ldx, q, ldq, s, lds},
                       WArgs{w, N, KB, ldw, qw, ldqw, sw, nullptr, 0, nullptr}, w_blocks);
}

}  // namespace fp8bs
