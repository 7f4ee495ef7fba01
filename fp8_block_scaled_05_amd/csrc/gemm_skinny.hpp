// Block-scaled FP8 GEMM for few rows (M up to a few tiles of 16..64): the
// weight stream from HBM is the whole cost, so the kernel is built to keep
// many weight bytes in flight.  Same arithmetic as gemm_kernel.hpp (one
// V_MFMA_F32_16X16X128_F8F6F4 per 16x16 tile and 128-K group, FP32
// promotion by S_A * S_W once per group; pages: "Advantages of using FP8 for
// GEMM operations in DeepSeek-V3", items 1 and 5; "How the unified E4M3
// format adds to DeepSeek-V3's efficiency", section "Enhanced numerical
// stability").
//
// Layout of the work: a workgroup owns BN = WAVES*FN*16 output columns and
// BM rows; each wave owns FN 16-column tiles.  The weight tile, the
// activation tile and both scale sets of every K group go HBM->LDS by direct
// buffer_load ... lds into one of DEPTH stages (distinct LDS arrays).  Groups
// are fetched in batches, so each weight row is read BATCH*128 contiguous
// bytes at a time, and NBATCH-1 batches stay in flight (vmcnt retires in
// order, so the waits are per batch).  Workgroups are small enough to keep
// every one of them resident, so the whole weight matrix streams at once.
#pragma once

#include "gemm_kernel.hpp"

namespace fp8bs {
namespace gemm {

template <int BM_, int FN_, int WAVES_, int BATCH_, int NBATCH_>
struct SkinnyCfg {
  static constexpr int BM = BM_, FN = FN_, NWAVES = WAVES_;
  // K groups are fetched in batches of BATCH; NBATCH batches are resident
  // (one being consumed, NBATCH-1 in flight); DEPTH = K groups resident
  static constexpr int BATCH = BATCH_, NBATCH = NBATCH_, DEPTH = BATCH * NBATCH;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int FM = BM / 16;
  static constexpr int BN = NWAVES * FN * 16;
  static constexpr int SA_LOADS = (BM + 63) / 64;
  static constexpr int A_LOADS = (BM / 8 + NWAVES - 1) / NWAVES;   // 1 KB each
  static constexpr bool A_DUMMY = A_LOADS * NWAVES * 8 > BM;
  static constexpr int B_LOADS = (BN / 8 + NWAVES - 1) / NWAVES;   // 1 KB each
  static_assert(B_LOADS * NWAVES * 8 == BN, "weight rows must split evenly over waves");
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * 128;
  static constexpr int SA_OFF = B_OFF + BN * 128;
  static constexpr int SB_OFF = SA_OFF + SA_LOADS * 256;
  static constexpr int DUMMY_OFF = SB_OFF + 256;                    // never read
  static constexpr int STAGE_BYTES = DUMMY_OFF + (A_DUMMY ? 1024 : 256);
  // per-wave copies of one K group, padded so every wave issues the same count
  static constexpr int SCALE_LOADS = (SA_LOADS + 1 + NWAVES - 1) / NWAVES;
  static constexpr int GROUP_OPS = A_LOADS + SCALE_LOADS + B_LOADS;
  static constexpr int WAIT_OPS = (NBATCH - 2) * BATCH * GROUP_OPS;
  static_assert(BM % 16 == 0 && BM <= 128, "BM");
  static_assert(FN * 16 <= 128 && 128 % (FN * 16) == 0, "a wave's columns share one weight block");
  static_assert(NBATCH >= 2 && DEPTH <= 12, "pipeline depth");
  static_assert(WAIT_OPS < 64, "vmcnt range");
  static_assert(DEPTH * STAGE_BYTES <= 160 * 1024, "LDS budget");
};

template <class C, bool OUT_BF16>
__device__ __forceinline__ void skinny_body(const GemmArgs& p) {
  // One distinct LDS array per pipeline stage, so that the compiler can tell
  // the stages apart when it tracks the outstanding direct-to-LDS copies.
#define FP8BS_SKINNY_STAGE(I) \
  __shared__ __attribute__((aligned(16))) uint8_t st##I[C::DEPTH > I ? C::STAGE_BYTES : 16];
  FP8BS_SKINNY_STAGE(0) FP8BS_SKINNY_STAGE(1) FP8BS_SKINNY_STAGE(2) FP8BS_SKINNY_STAGE(3)
  FP8BS_SKINNY_STAGE(4) FP8BS_SKINNY_STAGE(5) FP8BS_SKINNY_STAGE(6) FP8BS_SKINNY_STAGE(7)
  FP8BS_SKINNY_STAGE(8) FP8BS_SKINNY_STAGE(9) FP8BS_SKINNY_STAGE(10) FP8BS_SKINNY_STAGE(11)
#undef FP8BS_SKINNY_STAGE
  auto stage = [&](auto U) -> uint8_t* {
    constexpr int u = decltype(U)::value;
    if constexpr (u == 0) return st0;
    else if constexpr (u == 1) return st1;
    else if constexpr (u == 2) return st2;
    else if constexpr (u == 3) return st3;
    else if constexpr (u == 4) return st4;
    else if constexpr (u == 5) return st5;
    else if constexpr (u == 6) return st6;
    else if constexpr (u == 7) return st7;
    else if constexpr (u == 8) return st8;
    else if constexpr (u == 9) return st9;
    else if constexpr (u == 10) return st10;
    else return st11;
  };
  const int64_t KB = p.K / 128;
  const int64_t NB = (p.N + 127) / 128;
  const int64_t NT = (p.N + C::BN - 1) / C::BN;
  const int64_t tn = blockIdx.x % NT, tm = blockIdx.x / NT;
  const int64_t row0 = tm * C::BM, col0 = tn * C::BN;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int rows_a = (int)((p.M - row0) < C::BM ? (p.M - row0) : C::BM);  // >= 1

  // stage copies: A rows (swizzled like the main kernel), S_A, S_W
  uint32_t a_off[C::A_LOADS];
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int rbase = (wave * C::A_LOADS + j) * 8;
    const int r = rbase + (lane >> 3);
    const int rr = r < rows_a ? r : rows_a - 1;
    a_off[j] = (uint32_t)rr * (uint32_t)p.lda + ((lane & 7) ^ lds_swizzle(r)) * 16;
  }
  uint32_t s_off[C::SCALE_LOADS];
#pragma unroll
  for (int s = 0; s < C::SCALE_LOADS; ++s) {
    const int id = wave + s * C::NWAVES;
    if (id < C::SA_LOADS) {
      const int r = id * 64 + lane;
      s_off[s] = (uint32_t)(r < rows_a ? r : rows_a - 1) * 4;
    } else {
      const int64_t nbl = NB - 1 - col0 / 128;
      s_off[s] = (uint32_t)((lane < nbl ? lane : (int)nbl) * KB) * 4;
    }
  }
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + row0 * p.lda);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sa + row0);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(p.sb + (col0 / 128) * KB);

  // weight rows of the tile (swizzled like the activation rows)
  const int64_t wcol0 = col0 + wave * C::FN * 16;
  const int rows_b = (int)((p.N - col0) < C::BN ? (p.N - col0) : C::BN);  // >= 1
  uint32_t b_off[C::B_LOADS];
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int rbase = (wave * C::B_LOADS + j) * 8;
    const int r = rbase + (lane >> 3);
    const int rr = r < rows_b ? r : rows_b - 1;
    b_off[j] = (uint32_t)rr * (uint32_t)p.ldb + ((lane & 7) ^ lds_swizzle(r)) * 16;
  }
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.b + col0 * p.ldb);

  // all copies of K group kb into LDS stage U = kb % DEPTH
  auto issue_group = [&](auto U, int64_t kb) {
    uint8_t* st = stage(U);
#pragma unroll
    for (int s = 0; s < C::SCALE_LOADS; ++s) {
      const int id = wave + s * C::NWAVES;
      const bool is_sa = id < C::SA_LOADS;
      const int dst = is_sa ? C::SA_OFF + id * 256 : (id == C::SA_LOADS ? C::SB_OFF : C::DUMMY_OFF);
      const int soff = is_sa ? (int)(kb * p.ldsa * 4) : (int)(kb * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_sa ? rsa : rsb, (lds_void*)(st + dst), 4,
                                               s_off[s], soff, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::A_LOADS; ++j) {
      const int rbase = (wave * C::A_LOADS + j) * 8;
      // copies past the tile height land in the never-read slot
      uint8_t* dst = rbase < C::BM ? st + rbase * 128 : st + C::DUMMY_OFF;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)dst, 16, a_off[j],
                                               (int)(kb * 128), 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j) {
      const int rbase = (wave * C::B_LOADS + j) * 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + C::B_OFF + rbase * 128), 16,
                                               b_off[j], (int)(kb * 128), 0, 0);
    }
  };

  v4f acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int slot0 = (2 * g4) ^ lds_swizzle(l16);
  const int nb_local = (int)(wcol0 / 128 - col0 / 128);
  auto compute = [&](auto U) {
    const uint8_t* st = stage(U);
    const float sbv = reinterpret_cast<const float*>(st + C::SB_OFF)[nb_local];
    const float* sa = reinterpret_cast<const float*>(st + C::SA_OFF) + 4 * g4;
    v8i bf[C::FN];
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      bf[j] = load_frag(st, C::B_OFF + (wave * C::FN * 16 + 16 * j + l16) * 128 + slot0 * 16,
                        C::B_OFF + (wave * C::FN * 16 + 16 * j + l16) * 128 + (slot0 ^ 1) * 16,
                        0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const v8i af = load_frag(st, C::A_OFF + (16 * i + l16) * 128 + slot0 * 16,
                               C::A_OFF + (16 * i + l16) * 128 + (slot0 ^ 1) * 16, 0);
      const float4 s4 = *reinterpret_cast<const float4*>(sa + 16 * i);
      const float w0 = s4.x * sbv, w1 = s4.y * sbv, w2 = s4.z * sbv, w3 = s4.w * sbv;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af, bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc[i][j][0] = __builtin_fmaf(part[0], w0, acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(part[1], w1, acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(part[2], w2, acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(part[3], w3, acc[i][j][3]);
      }
    }
  };

  // Batches of BATCH groups are issued together (one wait and one barrier
  // per batch).  At the start of batch b every wave waits until only the
  // NBATCH-2 batches issued after b are in flight (vmcnt retires in order, so
  // batch b is then complete), meets the others at a barrier (all copies of
  // batch b visible; all reads of batch b-1's stages done), refills batch
  // b-1's stages and registers with batch b+NBATCH-1, then computes batch b.
  const int64_t NBK = (KB + C::BATCH - 1) / C::BATCH;  // batches
  // FULL: every group of the batch exists (no per-group guard; the steady
  // state must be branch-free so the compiler keeps precise copy tracking)
  auto issue_batch = [&](auto BI, auto FULL, int64_t b) {  // BI = b % NBATCH
    constexpr int bi = decltype(BI)::value;
    static_for<0, C::BATCH>([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int64_t kb = b * C::BATCH + g;
      if (decltype(FULL)::value || kb < KB)
        issue_group(std::integral_constant<int, bi * C::BATCH + g>{}, kb);
    });
  };
  using T = std::true_type;
  using F = std::false_type;
  static_for<0, C::NBATCH - 1>([&](auto BI) {
    if (decltype(BI)::value < NBK) issue_batch(BI, F{}, decltype(BI)::value);
  });

  auto run_batch = [&](auto BI, auto STEADY, int64_t b) {
    constexpr int bi = decltype(BI)::value;
    constexpr bool steady = decltype(STEADY)::value;
    if constexpr (steady) {
      wait_vmcnt<C::WAIT_OPS>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    constexpr int nxt = (bi + C::NBATCH - 1) % C::NBATCH;
    if constexpr (steady) {
      issue_batch(std::integral_constant<int, nxt>{}, T{}, b + C::NBATCH - 1);
    } else if (b + C::NBATCH - 1 < NBK) {
      issue_batch(std::integral_constant<int, nxt>{}, F{}, b + C::NBATCH - 1);
    }
    static_for<0, C::BATCH>([&](auto G) {
      constexpr int g = decltype(G)::value;
      if (steady || b * C::BATCH + g < KB)
        compute(std::integral_constant<int, bi * C::BATCH + g>{});
    });
  };

  int64_t b = 0;
  // steady state: every batch of the iteration is full and refills a full batch
  for (; (b + 2 * C::NBATCH - 1) * C::BATCH <= KB; b += C::NBATCH)
    static_for<0, C::NBATCH>([&](auto BI) { run_batch(BI, T{}, b + decltype(BI)::value); });
  static_for<0, 2 * C::NBATCH - 1>([&](auto U) {
    constexpr int u = decltype(U)::value;
    if (b + u < NBK) run_batch(std::integral_constant<int, u % C::NBATCH>{}, F{}, b + u);
  });

#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int64_t col = wcol0 + 16 * j + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + 16 * i + 4 * g4 + r;
        if (row < p.M && col < p.N) {
          if constexpr (OUT_BF16) {
            reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] = f32_to_bf16_rne(acc[i][j][r]);
          } else {
            reinterpret_cast<float*>(p.c)[row * p.ldc + col] = acc[i][j][r];
          }
        }
      }
    }
  }
}

template <class C, bool OUT_BF16>
__global__ __launch_bounds__(C::THREADS) void skinny_gemm_kernel(GemmArgs p) {
#if defined(__HIP_DEVICE_COMPILE__)
  skinny_body<C, OUT_BF16>(p);
#endif
}

template <class C>
hipError_t launch_skinny(const GemmArgs& args, bool out_bf16, hipStream_t stream) {
  const int64_t NT = (args.N + C::BN - 1) / C::BN;
  const int64_t MT = (args.M + C::BM - 1) / C::BM;
  const int64_t blocks = MT * NT;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (out_bf16) {
    hipLaunchKernelGGL((skinny_gemm_kernel<C, true>), dim3((unsigned)blocks), dim3(C::THREADS),
                       0, stream, args);
  } else {
    hipLaunchKernelGGL((skinny_gemm_kernel<C, false>), dim3((unsigned)blocks), dim3(C::THREADS),
                       0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace fp8bs
