// Few-row block-scaled FP8 GEMM for gfx950 (M <= 64: decode-like shapes),
// with the activation quantized inside the kernel for M <= 16.
//
// C[M][N] = A . W^T.  With few rows of A the time is the stream of W's E4M3
// codes from HBM (one byte per weight, read once), so both kernels here are
// built around that stream: workgroup b owns R consecutive rows of W
// (R = 8 RC, e.g. 72 for N = 18432 on 256 compute units: one workgroup per
// compute unit, every weight byte read once) over the whole K, copied
// HBM->LDS by direct buffer loads.  One V_MFMA_F32_16X16X128_F8F6F4 per
// 16x16 output tile and 128-K group with W as its first operand, promoted
// into FP32 by S_A(m, kb) * S_W(n / 128, kb) ("Advantages of using FP8 for
// GEMM operations in DeepSeek-V3", item 5; "How the unified E4M3 format
// adds to DeepSeek-V3's efficiency", section "Enhanced numerical
// stability").  The weight-block scales are read through the scalar cache:
// as vector loads they would join the in-order count of the tile copies,
// and the wait for them would drain every copy in flight.
//
// - few_rows_kteam_kernel (M <= 32): the four waves take the K groups in
//   turn (wave w: groups w, w + 4, ...), each with a private ring of four
//   LDS stages, so no barrier is needed until the waves' partial sums are
//   added in LDS (in a fixed order).  Lane (g, l) supplies 32 K values of A
//   row 16 j + l for each 16-row tile j of A.  With a bf16 A (FUSED, M <=
//   16) each wave loads those values and quantizes them in registers by the
//   online 1x128 rule ("How online quantization in DeepSeek-V3 differs from
//   delayed quantization", item 1; "Advantages of using FP8 for GEMM
//   operations in DeepSeek-V3", item 7) with the standalone quantizer's
//   arithmetic, so codes and scales are that kernel's bit for bit.  Every
//   workgroup quantizes all of A, which at M <= 16 costs less than a
//   separate quantizer launch; at 32 and 64 rows the same VALU work per
//   compute unit did not hide under the stream and two launches measured
//   faster, so larger bf16 A is quantized first.
// - few_rows_shared_kernel (32 < M <= 64, E4M3 A): the four waves share
//   each K group's stage, which also holds the group's A codes and scales,
//   and wave w takes A rows 16 w .. 16 w + 15.

// Built with -mllvm -amdgpu-mfma-vgpr-form (build.py): one wave per SIMD may
// hold 512 registers, and the compiler would otherwise write every MFMA
// result to accumulation registers that each promotion must copy out first
// (four extra VALU instructions per MFMA).

#include "gemm_kernel.hpp"

namespace fp8bs {

namespace {

using gemm::lds_swizzle;
using gemm::make_rsrc;
using gemm::wait_vmcnt;

constexpr int kWaves = 4;
constexpr int kStages = 4;

template <int RC, int MT, bool FUSED>
struct FewCfg {
  static constexpr int R = 8 * RC;                  // weight rows per workgroup
  static constexpr int RT = (R + 15) / 16;          // 16-row MFMA tiles of W
  static constexpr int WAVE_BYTES = RT * 16 * 128;  // one wave's share of a stage
  static constexpr int STAGE_BYTES = kWaves * WAVE_BYTES;
  // vector-memory operations per K group per wave: RC tile copies, then the
  // A loads (bf16: 4 x 16 bytes per tile of A; codes: 2 x 16 bytes and the
  // scale)
  static constexpr int NA = FUSED ? 4 * MT : 3 * MT;
  // A loads in flight ahead of their use: two groups when their registers
  // are few, one for the bf16 A of four tiles
  static constexpr int ADIST = (FUSED && MT > 2) ? 1 : 2;
  static_assert(kStages * STAGE_BYTES <= 160 * 1024, "LDS budget");
  static_assert(ADIST * RC + (ADIST - 1) * NA <= 63, "vmcnt range");
};

// The bf16 A values of one lane for one 16-row tile of A and K group (FUSED),
// or its E4M3 codes and scale.
template <bool FUSED>
struct ARegs;
template <>
struct ARegs<true> {
  u32x4 v[4];
};
template <>
struct ARegs<false> {
  u32x4 v[2];
  float s;
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Wave-uniform read-only float through the scalar cache.  A vector load
// would join the in-order vmcnt stream of the tile copies, and the wait for
// its value would drain every copy in flight.
__device__ __forceinline__ float scalar_ld(const float* p) {
  return *(const __attribute__((address_space(4))) float*)(p);
}

// Largest magnitude of the 32 bf16 values of a lane, as float32: finite
// bf16 magnitudes order like their 15-bit patterns, so the maximum is taken
// on the bits with packed 16-bit integer maxima.
__device__ __forceinline__ float absmax32_bf16(const u32x4 (&v)[4]) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t d[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, d[e] & 0x7FFF7FFFu));
  }
  const uint32_t b = m.x > m.y ? m.x : m.y;
  return __uint_as_float(b << 16);
}

// E4M3 codes of one lane's 32 bf16 values of an A tile (K values 32 g ..
// 32 g + 31 of one row) and the tile's scale s; the row's other 96 values
// are on lanes lane ^ 16, ^ 32, ^ 48.  The online 1x128 rule with the
// standalone quantizer's arithmetic (amax, group_scale, RN32(x * r), RNE
// convert), so codes and scale are that kernel's bit for bit -- except that
// the clamp to +-448 before the convert is left out: with r = RN32(448/a)
// and |x| <= a, every finite input gives |x r| <= 448.0000534, and the bare
// convert takes [448, 464) to the code of 448 (both checked exhaustively),
// so the clamp changes nothing here (it only matters for NaN and infinite
// input, which is outside the contract).
// `between(k)` runs after the scale (k = 0) and after each quarter of the
// converts (k = 1..3): a caller interleaves its copies with this VALU work.
template <class F>
__device__ __forceinline__ v8i quant_tile32(const u32x4 (&v)[4], float& s, F&& between) {
  float amax = absmax32_bf16(v);
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  float r;
  group_scale(amax, s, r);
  v8i out;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    between(q);
    const uint32_t d[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
          bf16_lo(d[2 * h]) * r, bf16_hi(d[2 * h]) * r, 0, false);
      w[h] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(
          bf16_lo(d[2 * h + 1]) * r, bf16_hi(d[2 * h + 1]) * r, (int)lo, true);
    }
    out[2 * q] = (int)w[0];
    out[2 * q + 1] = (int)w[1];
  }
  return out;
}

struct FewArgs {
  const void* a;  // FUSED: bf16 [M][lda]; else E4M3 codes [M][lda]
  int64_t lda;
  float* sa;      // FUSED: optional output; else input.  s(m, kb) at sa[kb*ldsa + m]
  int64_t ldsa;
  const uint8_t* b;  // E4M3 [N][ldb]
  int64_t ldb;
  const float* sb;   // S_W [N/128][K/128]
  void* c;           // fp32 or bf16 [M][ldc]
  int64_t ldc;
  int64_t M, N, K;
  int out_bf16;
};

template <int RC, int MT, bool FUSED>
__global__ __launch_bounds__(kWaves * 64) void few_rows_kteam_kernel(FewArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = FewCfg<RC, MT, FUSED>;
  constexpr int RT = C::RT;
  __shared__ __attribute__((aligned(16))) uint8_t st0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t st1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t st2[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t st3[C::STAGE_BYTES];
  uint8_t* const stages[kStages] = {st0, st1, st2, st3};

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * C::R;
  const int nrows = (int)((p.N - row0) < C::R ? (p.N - row0) : C::R);  // >= 1
  const int64_t KB = p.K / 128;
  // this wave's K groups: wave, wave + 4, ... (T of them)
  const int T = KB > wave ? (int)((KB - wave + kWaves - 1) / kWaves) : 0;

  v4f acc[RT][MT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  if (T > 0) {
    // --- per-lane constants ---
    // tile copies: copy c fills stage rows 8c .. 8c + 7 (rows past the
    // workgroup's last row repeat it); 16-byte chunk `slot` of LDS row r
    // holds K chunk slot ^ lds_swizzle(r)
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.b + row0 * p.ldb);
    uint32_t voff[RC];
#pragma unroll
    for (int c = 0; c < RC; ++c) {
      const int r = 8 * c + (lane >> 3);
      const int rr = r < nrows ? r : nrows - 1;
      voff[c] = (uint32_t)rr * (uint32_t)p.ldb + (uint32_t)(((lane & 7) ^ lds_swizzle(r)) * 16);
    }
    // W fragment reads: row 16 i + l16, K chunks 2g and 2g + 1
    const int slot0 = (2 * g) ^ lds_swizzle(l16);
    int f_lo = wave * C::WAVE_BYTES + l16 * 128 + slot0 * 16;
    int f_hi = wave * C::WAVE_BYTES + l16 * 128 + (slot0 ^ 1) * 16;
    asm volatile("" : "+v"(f_lo), "+v"(f_hi));
    // A rows of this lane (rows past M repeat the last)
    int64_t arow[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int64_t m = 16 * j + l16;
      arow[j] = m < p.M ? m : p.M - 1;
    }
    // weight-block scales: the workgroup's rows span blocks nb_lo .. nb_hi
    // (at most two); row tile i's lane rows 16 i + 4 g .. + 3 share one
    const int64_t NB = (p.N + 127) / 128;
    const int64_t nb_lo = row0 / 128;
    int64_t nb_hi = (row0 + C::R - 1) / 128;
    nb_hi = nb_hi < NB ? nb_hi : NB - 1;
    bool use_hi[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) use_hi[i] = (row0 + 16 * i + 4 * g) / 128 != nb_lo;
    const float* sw_lo = p.sb + nb_lo * KB;
    const float* sw_hi = p.sb + nb_hi * KB;

    const int last_kb = wave + kWaves * (T - 1);
    auto kb_of = [&](int t) -> int { return t < T ? wave + kWaves * t : last_kb; };

    // copies [c0, c1) of group t into stage st
    auto issue_w = [&](int t, uint8_t* st, int c0, int c1) {
      const int kb = kb_of(t);
#pragma unroll
      for (int c = 0; c < RC; ++c) {
        if (c < c0 || c >= c1) continue;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wrs, (gemm::lds_void*)(st + wave * C::WAVE_BYTES + c * 1024), 16, voff[c], kb * 128,
            0, 0);
      }
    };
    // A values of group t for tile j of A into `ar`
    auto issue_a_tile = [&](int t, int j, ARegs<FUSED>& ar) {
      const int64_t kb = kb_of(t);
      if constexpr (FUSED) {
        const u32x4* src = reinterpret_cast<const u32x4*>(
            static_cast<const uint16_t*>(p.a) + arow[j] * p.lda + kb * 128 + 32 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) ar.v[q] = src[q];
      } else {
        const u32x4* src = reinterpret_cast<const u32x4*>(
            static_cast<const uint8_t*>(p.a) + arow[j] * p.lda + kb * 128 + 32 * g);
        ar.v[0] = src[0];
        ar.v[1] = src[1];
        ar.s = p.sa[kb * p.ldsa + arow[j]];
      }
    };
    auto issue_a = [&](int t, ARegs<FUSED> (&ar)[MT]) {
#pragma unroll
      for (int j = 0; j < MT; ++j) issue_a_tile(t, j, ar[j]);
    };

    ARegs<FUSED> abuf[C::ADIST][MT];

    // One K group t (stage U = t mod 4, A buffer B = t mod ADIST).  Wait for
    // its copies and A values; read the stage's W fragments; then, tile by
    // tile of A: form the MFMA operand (quantizing a bf16 A), refill that
    // tile's registers with group t + ADIST, and run the MFMAs and their
    // FP32 promotion; last, the copies of group t + 3 into the stage read
    // one group ago.  Every group issues the same operations (past the last
    // group they repeat it, into a stage and registers nobody reads), so
    // the wait counts are constants: when group t's A values have landed,
    // everything issued after them may still be in flight -- the copies of
    // group t + 3 - ADIST and, for each group in between, its A loads and
    // copies (ADIST RC + (ADIST - 1) NA operations; group t's copies were
    // issued before its A loads).
    auto step = [&](int t, auto U_, auto B_) {
      constexpr int U = decltype(U_)::value, Bf = decltype(B_)::value;
      // keep each group's work inside its step (no motion across groups,
      // which would hold two groups' operands in registers)
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<C::ADIST * RC + (C::ADIST - 1) * C::NA>();
      const int kb = kb_of(t);
      const float swl = scalar_ld(sw_lo + kb), swh = scalar_ld(sw_hi + kb);
      const uint8_t* st = stages[U];
      v8i wf[RT];
#pragma unroll
      for (int i = 0; i < RT; ++i) wf[i] = gemm::load_frag(st, f_lo, f_hi, i * 2048);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        v8i af;
        float fa;
        if constexpr (FUSED) {
          float s;
          af = quant_tile32(abuf[Bf][j].v, s, [](int) {});
          fa = s;
          if (p.sa != nullptr && blockIdx.x == 0 && g == 0 && 16 * j + l16 < p.M)
            p.sa[(int64_t)kb * p.ldsa + 16 * j + l16] = s;
        } else {
          const ARegs<false>& ar = abuf[Bf][j];
          af = __builtin_shufflevector((gemm::v4i)ar.v[0], (gemm::v4i)ar.v[1], 0, 1, 2, 3, 4, 5,
                                       6, 7);
          fa = ar.s;
        }
        issue_a_tile(t + C::ADIST, j, abuf[Bf][j]);
        // the promotion of row tile i follows the MFMA of row tile i + 1;
        // with the last tile of A, the copies of group t + 3 (into the stage
        // read one group ago) are spread over the MFMAs, after every A load
        // of the step as the wait counts assume
        constexpr int PW = (RC + RT - 1) / RT;
        v4f prev;
#pragma unroll
        for (int i = 0; i <= RT; ++i) {
          v4f cur;
          if (i < RT) {
            cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                wf[i], af, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            if (j == MT - 1) issue_w(t + 3, stages[(U + 3) % kStages], i * PW, (i + 1) * PW);
          }
          if (i > 0) {
            const float f = fa * (use_hi[i - 1] ? swh : swl);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[i - 1][j][r] = __builtin_fmaf(prev[r], f, acc[i - 1][j][r]);
          }
          if (i < RT) prev = cur;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: the order in which steps -3, -2, -1 would have issued
    // (A loads of group t + ADIST, then copies of group t + 3)
    if constexpr (C::ADIST == 2) {
      issue_w(0, stages[0], 0, RC);
      issue_a(0, abuf[0]);
      issue_w(1, stages[1], 0, RC);
      issue_a(1, abuf[1]);
      issue_w(2, stages[2], 0, RC);
    } else {
      issue_w(0, stages[0], 0, RC);
      issue_w(1, stages[1], 0, RC);
      issue_a(0, abuf[0]);
      issue_w(2, stages[2], 0, RC);
    }
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    constexpr bool D2 = C::ADIST == 2;
    int t = 0;
    for (; t + 4 <= T; t += 4) {
      step(t, I0{}, I0{});
      step(t + 1, I1{}, std::integral_constant<int, D2 ? 1 : 0>{});
      step(t + 2, I2{}, I0{});
      step(t + 3, I3{}, std::integral_constant<int, D2 ? 1 : 0>{});
    }
    if (t < T) step(t, I0{}, I0{});
    if (t + 1 < T) step(t + 1, I1{}, std::integral_constant<int, D2 ? 1 : 0>{});
    if (t + 2 < T) step(t + 2, I2{}, I0{});
    wait_vmcnt<0>();
  }

  // --- the waves' partial sums, added in LDS in wave order, then stored ---
  // rounds of up to NR tiles: every wave writes its NR tiles (1 KB each) to
  // stage 0, then wave w adds up the tiles q = w, w + 4, ... of the round
  constexpr int NQ = RT * MT;
  constexpr int NR = (C::STAGE_BYTES / (kWaves * 1024)) < NQ ? C::STAGE_BYTES / (kWaves * 1024)
                                                              : NQ;
  float* const red = reinterpret_cast<float*>(st0);
  const bool vec = p.ldc % 4 == 0 &&
                   reinterpret_cast<uintptr_t>(p.c) % (p.out_bf16 ? 8 : 16) == 0;
#pragma unroll
  for (int q0 = 0; q0 < NQ; q0 += NR) {
    __syncthreads();
#pragma unroll
    for (int qq = 0; qq < NR; ++qq) {
      const int q = q0 + qq;
      if (q < NQ)
        *reinterpret_cast<v4f*>(red + ((wave * NR + qq) * 64 + lane) * 4) =
            acc[q / MT][q % MT];
    }
    __syncthreads();
    for (int qq = wave; qq < NR && q0 + qq < NQ; qq += kWaves) {
      const int q = q0 + qq, i = q / MT, j = q % MT;
      v4f sum = *reinterpret_cast<const v4f*>(red + (qq * 64 + lane) * 4);
#pragma unroll
      for (int w = 1; w < kWaves; ++w)
        sum += *reinterpret_cast<const v4f*>(red + ((w * NR + qq) * 64 + lane) * 4);
      const int64_t m = 16 * j + l16;
      const int nl = 16 * i + 4 * g;  // first of the lane's 4 output columns
      if (m >= p.M || nl >= nrows) continue;
      const int64_t n = row0 + nl;
      if (p.out_bf16) {
        uint16_t* dst = static_cast<uint16_t*>(p.c) + m * p.ldc + n;
        if (vec && nl + 4 <= nrows) {
          const uint32_t lo = bf16x2_rne(sum[0], sum[1]);
          const uint32_t hi = bf16x2_rne(sum[2], sum[3]);
          *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
        } else {
          for (int r = 0; r < 4 && nl + r < nrows; ++r) dst[r] = f32_to_bf16_rne(sum[r]);
        }
      } else {
        float* dst = static_cast<float*>(p.c) + m * p.ldc + n;
        if (vec && nl + 4 <= nrows) {
          *reinterpret_cast<v4f*>(dst) = sum;
        } else {
          for (int r = 0; r < 4 && nl + r < nrows; ++r) dst[r] = sum[r];
        }
      }
    }
  }
#endif
}

// 32 < M <= 64 (E4M3 A): the four waves share each K group's stage and wave
// w takes the 16 rows 16 w .. 16 w + 15 of A (rows past M repeat the last).
// A stage holds the group's R weight rows, its 64 rows of A codes and their
// 64 scales, all copied HBM->LDS by direct buffer loads, so no operand
// waits in registers and the ring is deep (S stages, S - 1 groups in
// flight).  Each wave issues its share of a group's copies (the 1-KB blocks
// b = 4 s + w; the last block again where the count does not divide, the
// same bytes to the same place) and one scale copy.  One barrier per group:
// after it every copy of the group has landed (each wave waited for its
// own) and every wave has left the previous group's stage, which is
// refilled next; that refill is spread over the group's MFMAs (a burst of
// copies stalls the wave at issue).
template <int RC>
struct SharedCfg {
  static constexpr int R = 8 * RC;
  static constexpr int RT = (R + 15) / 16;
  static constexpr int A_OFF = RT * 16 * 128;  // the last tile's rows past R are never copied
  static constexpr int SC_OFF = A_OFF + 64 * 128;
  static constexpr int STAGE_BYTES = SC_OFF + 256;
  static constexpr int S0 = (160 * 1024) / STAGE_BYTES;
  static constexpr int S = S0 > 8 ? 8 : S0;
  static constexpr int NBLK = RC + 8;                       // 1-KB copies: W, then A codes
  static constexpr int BPW = (NBLK + kWaves - 1) / kWaves;  // per wave
  static constexpr int CPW = BPW + 1;                       // plus the scale copy
  static_assert(S >= 3, "stage ring");
  static_assert((S - 2) * CPW <= 63, "vmcnt range");
};

template <int RC>
__global__ __launch_bounds__(kWaves * 64) void few_rows_shared_kernel(FewArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = SharedCfg<RC>;
  constexpr int RT = C::RT, S = C::S;
  constexpr int SB = C::STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st2[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st3[S > 3 ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st4[S > 4 ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st5[S > 5 ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st6[S > 6 ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st7[S > 7 ? SB : 16];
  uint8_t* const stages[8] = {st0, st1, st2, st3, st4, st5, st6, st7};

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t row0 = (int64_t)blockIdx.x * C::R;
  const int nrows = (int)((p.N - row0) < C::R ? (p.N - row0) : C::R);  // >= 1
  const int KB = (int)(p.K / 128);

  // copies: slot s of this wave is block b = 4 s + wave; blocks [0, RC) are
  // 8 weight rows, the next 8 are 8 rows of A codes each
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(p.b + row0 * p.ldb);
  const __amdgpu_buffer_rsrc_t ars = make_rsrc(p.a);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.sa);
  uint32_t voff[C::BPW];
  int ldsoff[C::BPW];
  bool is_w[C::BPW];
#pragma unroll
  for (int sl = 0; sl < C::BPW; ++sl) {
    int b = 4 * sl + wave;
    b = b < C::NBLK ? b : C::NBLK - 1;
    is_w[sl] = b < RC;
    if (b < RC) {
      const int r = 8 * b + (lane >> 3);
      const int rr = r < nrows ? r : nrows - 1;
      voff[sl] = (uint32_t)rr * (uint32_t)p.ldb + (uint32_t)(((lane & 7) ^ lds_swizzle(r)) * 16);
      ldsoff[sl] = b * 1024;
    } else {
      const int r = 8 * (b - RC) + (lane >> 3);
      const int64_t m = r < p.M ? r : p.M - 1;
      voff[sl] = (uint32_t)(m * p.lda) + (uint32_t)(((lane & 7) ^ lds_swizzle(r)) * 16);
      ldsoff[sl] = C::A_OFF + (b - RC) * 1024;
    }
  }
  // every wave copies the group's 64 activation scales (4 bytes per lane)
  const uint32_t soff = (uint32_t)((lane < p.M ? lane : p.M - 1) * 4);

  // this wave's copies [s0, s1) of group t into stage st (slot BPW: the
  // scale copy); past the last group: the last group again
  auto issue = [&](int t, uint8_t* st, int s0, int s1) {
    const int kb = t < KB ? t : KB - 1;
#pragma unroll
    for (int sl = 0; sl < C::CPW; ++sl) {
      if (sl < s0 || sl >= s1) continue;
      if (sl < C::BPW) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_w[sl] ? wrs : ars,
                                                 (gemm::lds_void*)(st + ldsoff[sl]), 16,
                                                 voff[sl], kb * 128, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (gemm::lds_void*)(st + C::SC_OFF), 4, soff,
                                                 (int)(kb * p.ldsa * 4), 0, 0);
      }
    }
  };

  // per-lane LDS read offsets: weight row 16 i + l16 and A row 16 w + l16,
  // K chunks 2g and 2g + 1
  const int slot0 = (2 * g) ^ lds_swizzle(l16);
  const int ar = 16 * wave + l16;
  int f_lo = l16 * 128 + slot0 * 16;
  int f_hi = l16 * 128 + (slot0 ^ 1) * 16;
  int a_lo = C::A_OFF + ar * 128 + slot0 * 16;
  int a_hi = C::A_OFF + ar * 128 + (slot0 ^ 1) * 16;
  asm volatile("" : "+v"(f_lo), "+v"(f_hi), "+v"(a_lo), "+v"(a_hi));
  const int64_t NB = (p.N + 127) / 128;
  const int64_t nb_lo = row0 / 128;
  int64_t nb_hi = (row0 + C::R - 1) / 128;
  nb_hi = nb_hi < NB ? nb_hi : NB - 1;
  bool use_hi[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) use_hi[i] = (row0 + 16 * i + 4 * g) / 128 != nb_lo;
  const float* sw_lo = p.sb + nb_lo * KB;
  const float* sw_hi = p.sb + nb_hi * KB;

  v4f acc[RT];
#pragma unroll
  for (int i = 0; i < RT; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};

  // group t from stage U = t mod S: wait for this wave's copies of it (the
  // S - 2 later groups' stay in flight), meet the other waves, then the
  // MFMAs with the refill of the stage left one group ago (group t + S - 1)
  // spread over them
  auto step = [&](int t, auto U_) {
    constexpr int U = decltype(U_)::value;
    constexpr int PR = (C::CPW + RT - 1) / RT;
    __builtin_amdgcn_sched_barrier(0);
    gemm::barrier_after_vmcnt<(S - 2) * C::CPW>();
    uint8_t* const nxt = stages[(U + S - 1) % S];
    const uint8_t* st = stages[U];
    const float swl = scalar_ld(sw_lo + t), swh = scalar_ld(sw_hi + t);
    const v8i af = gemm::load_frag(st, a_lo, a_hi, 0);
    const float fa = reinterpret_cast<const float*>(st + C::SC_OFF)[ar];
    v4f prev;
#pragma unroll
    for (int i = 0; i <= RT; ++i) {
      v4f cur;
      if (i < RT) {
        const v8i wf = gemm::load_frag(st, f_lo, f_hi, i * 2048);
        cur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, af, v4f{0.f, 0.f, 0.f, 0.f},
                                                               0, 0, 0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue(t + S - 1, nxt, i * PR, (i + 1) * PR);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i > 0) {
        const float f = fa * (use_hi[i - 1] ? swh : swl);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i - 1][r] = __builtin_fmaf(prev[r], f, acc[i - 1][r]);
      }
      if (i < RT) prev = cur;
    }
  };

  // prologue: groups 0 .. S - 2
#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(u, stages[u], 0, C::CPW);
  int t = 0;
  for (; t + S <= KB; t += S) {
    static_for<0, S>([&](auto U) { step(t + decltype(U)::value, U); });
  }
  static_for<0, S - 1>([&](auto U) {
    if (t + decltype(U)::value < KB) step(t + decltype(U)::value, U);
  });
  wait_vmcnt<0>();

  // --- store: wave w holds C[16 w + l16][row0 + 16 i + 4 g + r] ---
  const int64_t m = ar;
  if (m < p.M) {
    const bool vec = p.ldc % 4 == 0 &&
                     reinterpret_cast<uintptr_t>(p.c) % (p.out_bf16 ? 8 : 16) == 0;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const int nl = 16 * i + 4 * g;
      if (nl >= nrows) continue;
      const int64_t n = row0 + nl;
      const v4f sum = acc[i];
      if (p.out_bf16) {
        uint16_t* dst = static_cast<uint16_t*>(p.c) + m * p.ldc + n;
        if (vec && nl + 4 <= nrows) {
          const uint32_t lo = bf16x2_rne(sum[0], sum[1]);
          const uint32_t hi = bf16x2_rne(sum[2], sum[3]);
          *reinterpret_cast<u32x2*>(dst) = u32x2{lo, hi};
        } else {
          for (int r = 0; r < 4 && nl + r < nrows; ++r) dst[r] = f32_to_bf16_rne(sum[r]);
        }
      } else {
        float* dst = static_cast<float*>(p.c) + m * p.ldc + n;
        if (vec && nl + 4 <= nrows) {
          *reinterpret_cast<v4f*>(dst) = sum;
        } else {
          for (int r = 0; r < 4 && nl + r < nrows; ++r) dst[r] = sum[r];
        }
      }
    }
  }
#endif
}

// Weight rows per workgroup (RC 8-row copies): the fewest that put the
// whole N on at most one workgroup per compute unit, from a fixed set.
template <int MT, bool FUSED>
hipError_t launch_mt(const FewArgs& p, int cus, hipStream_t stream) {
  const int64_t per = (p.N + cus - 1) / cus;
  auto go = [&](auto RC_) {
    constexpr int RC = decltype(RC_)::value;
    const int64_t blocks = (p.N + 8 * RC - 1) / (8 * RC);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    return launch_kernel(few_rows_kteam_kernel<RC, MT, FUSED>, dim3((unsigned)blocks),
                         dim3(kWaves * 64), stream, p);
  };
  if (per <= 8) return go(std::integral_constant<int, 1>{});
  if (per <= 24) return go(std::integral_constant<int, 3>{});
  return go(std::integral_constant<int, 9>{});
}

hipError_t launch_shared(const FewArgs& p, int cus, hipStream_t stream) {
  const int64_t per = (p.N + cus - 1) / cus;
  auto go = [&](auto RC_) {
    constexpr int RC = decltype(RC_)::value;
    const int64_t blocks = (p.N + 8 * RC - 1) / (8 * RC);
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    return launch_kernel(few_rows_shared_kernel<RC>, dim3((unsigned)blocks), dim3(kWaves * 64),
                         stream, p);
  };
  if (per <= 8) return go(std::integral_constant<int, 1>{});
  if (per <= 24) return go(std::integral_constant<int, 3>{});
  return go(std::integral_constant<int, 9>{});
}

}  // namespace

hipError_t launch_few_rows_gemm(const void* a, int64_t lda, float* sa, int64_t ldsa, bool fused,
                                const uint8_t* b, int64_t ldb, const float* sb, void* c,
                                int64_t ldc, bool out_bf16, int64_t M, int64_t N, int64_t K,
                                hipStream_t stream) {
  const FewArgs p{a, lda, sa, ldsa, b, ldb, sb, c, ldc, M, N, K, out_bf16 ? 1 : 0};
  const int cus = gemm::device_cus();
  if (cus <= 0) return hipErrorInvalidDevice;
  if (fused) {
    if (M > kFewRowsFused) return hipErrorInvalidValue;
    return launch_mt<1, true>(p, cus, stream);
  }
  if (M <= 16) return launch_mt<1, false>(p, cus, stream);
  if (M <= 32) return launch_mt<2, false>(p, cus, stream);
  if (M <= kFewRows) return launch_shared(p, cus, stream);
  return hipErrorInvalidValue;
}

}  // namespace fp8bs
