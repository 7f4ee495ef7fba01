// Block-scaled FP8 GEMM for gfx950 (dense and grouped/MoE).
//
// C = A . B^T with E4M3 operands.  For every 128-wide K group kb the kernel
// forms the FP8 x FP8 partial product of that group in FP32 (one
// V_MFMA_F32_16X16X128_F8F6F4 covers a 16x16 output tile's whole group) and
// promotes it into the FP32 running sum with one multiply-add by
// S_A(m,kb) * S_W(n/128,kb).  Pages: "Advantages of using FP8 for GEMM
// operations in DeepSeek-V3", items 1, 5 and 8 (FP8 GEMM for dense and MoE
// layers; partial results promoted to FP32 registers at fixed intervals of
// the accumulation); "How the unified E4M3 format adds to DeepSeek-V3's
// efficiency", section "Enhanced numerical stability".  The promotion
// interval is the 128-K group, where the scales change.
//
// Structure: 256 threads (4 waves, 2x2) per BMxBN output tile.  Each K group
// of A, B and the activation scales is copied HBM->LDS by direct
// global_load_lds_dwordx4 (no register staging) into one of two LDS stages
// while the other stage feeds the MFMAs.  LDS rows are 128 bytes; the eight
// 16-byte chunks of row r are stored XOR-swizzled by (r & 7) so that the
// 16 lanes reading one K chunk of 16 different rows hit different banks.
// The MFMA K order inside a lane (32 bytes = chunks 2g, 2g+1 for lane group
// g) is the same for A and B, so every product pairs matching K indices.

#include "device.hpp"
#include "internal.hpp"

namespace fp8bs {

namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kGroupM = 8;  // tile-rows per swizzle group (L2 reuse of B)

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0), other counters untouched
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <int ROWS>
__device__ __forceinline__ void issue_tile_rows(const uint8_t* __restrict__ base, int64_t ld,
                                                int64_t row0, int64_t row_end, int64_t kb,
                                                uint8_t* lds, int wave, int lane) {
  // ROWS x 128 bytes; a wave moves 8 rows (1 KB) per instruction.
  constexpr int kPerWave = ROWS / 32;
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int rbase = wave * (ROWS / 4) + 8 * j;
    const int r = rbase + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    int64_t grow = row0 + r;
    grow = grow < row_end ? grow : row_end - 1;
    const uint8_t* src = base + grow * ld + kb * 128 + chunk * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(lds + rbase * 128), 16, 0, 0);
  }
}

template <int BM>
__device__ __forceinline__ void issue_scales(const float* __restrict__ sa, int64_t ldsa,
                                             int64_t row0, int64_t row_end,
                                             const float* __restrict__ sb, int64_t nb0,
                                             int64_t nb_last, int64_t KB, int64_t kb,
                                             float* lds_sa, float* lds_sb, int wave, int lane) {
  // activation scales of the tile's BM rows for group kb (64 rows per wave)
  if (wave < BM / 64) {
    int64_t grow = row0 + wave * 64 + lane;
    grow = grow < row_end ? grow : row_end - 1;
    __builtin_amdgcn_global_load_lds((const void*)(sa + kb * ldsa + grow),
                                     (lds_void*)(lds_sa + wave * 64), 4, 0, 0);
  } else if (wave == BM / 64) {
    // weight-block scales of the tile's 128-column blocks for group kb
    int64_t nb = nb0 + lane;
    nb = nb < nb_last ? nb : nb_last;
    __builtin_amdgcn_global_load_lds((const void*)(sb + nb * KB + kb), (lds_void*)lds_sb, 4, 0, 0);
  }
}

template <int BM, int BN, bool GROUPED, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void block_gemm_kernel(GemmArgs p) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 16, FN = WN / 16;
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must share one weight block");

  // one LDS stage = [A: BM x 128 B | B: BN x 128 B | activation scales: BM fp32 |
  //                  weight-block scales: 64 fp32]
  static_assert(BM / 64 < 4, "one wave must be left to fetch the weight-block scales");
  constexpr int kStage = BM * 128 + BN * 128 + BM * 4 + 64 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t st1[kStage];
  uint8_t* const sA0 = st0;
  uint8_t* const sB0 = st0 + BM * 128;
  float* const sS0 = reinterpret_cast<float*>(st0 + BM * 128 + BN * 128);
  float* const sW0 = sS0 + BM;
  uint8_t* const sA1 = st1;
  uint8_t* const sB1 = st1 + BM * 128;
  float* const sS1 = reinterpret_cast<float*>(st1 + BM * 128 + BN * 128);
  float* const sW1 = sS1 + BM;

  const int64_t KB = p.K / 128;
  const int64_t NB = (p.N + 127) / 128;
  const int64_t NT = (p.N + BN - 1) / BN;
  const int64_t MT = GROUPED ? (p.M + BM - 1) / BM + p.G : (p.M + BM - 1) / BM;

  // Tile order: workgroups are dealt round-robin to the 8 XCDs; give each XCD
  // a contiguous run of tiles, and inside it walk kGroupM tile-rows before
  // moving along N so that concurrently resident tiles share A and B in L2.
  int64_t bid = blockIdx.x;
  const int64_t T = (int64_t)gridDim.x;
  if (T % 8 == 0) bid = (bid % 8) * (T / 8) + bid / 8;
  const int64_t per_group = (int64_t)kGroupM * NT;
  const int64_t first_m = (bid / per_group) * kGroupM;
  const int64_t gsz = (MT - first_m) < kGroupM ? (MT - first_m) : kGroupM;
  const int64_t in_grp = bid % per_group;
  const int64_t tm = first_m + in_grp % gsz;
  const int64_t tn = in_grp / gsz;

  int64_t row0, row_end;
  const uint8_t* __restrict__ bmat = p.b;
  const float* __restrict__ sbmat = p.sb;
  if constexpr (GROUPED) {
    const int32_t* __restrict__ off = p.group_offsets;
    int64_t seen = 0;
    int64_t g = -1, local = 0;
    for (int64_t gg = 0; gg < p.G; ++gg) {
      const int64_t cnt = ((int64_t)off[gg + 1] - off[gg] + BM - 1) / BM;
      if (tm < seen + cnt) {
        g = gg;
        local = tm - seen;
        break;
      }
      seen += cnt;
    }
    if (g < 0) return;  // beyond the last real tile (whole workgroup)
    row0 = off[g] + local * BM;
    row_end = off[g + 1];
    bmat += g * p.b_group_stride;
    sbmat += g * NB * KB;
  } else {
    row0 = tm * BM;
    row_end = p.M;
  }
  const int64_t col0 = tn * BN;

  // wave index in an SGPR so that per-wave values (the weight block index)
  // stay scalar and their loads go through the scalar cache
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int g4 = lane >> 4;      // K chunk pair / output row quad
  const int l16 = lane & 15;     // row of A fragment, column of B fragment / output
  const int slot0 = (2 * g4) ^ (lane & 7);
  const int slot1 = slot0 ^ 1;
  const int64_t nb0 = col0 / 128;
  const int nb_local = (wn * WN) / 128;  // this wave's weight block within the tile

  v4f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int64_t kb, uint8_t* la, uint8_t* lb, float* ls, float* lw) {
    issue_tile_rows<BM>(p.a, p.lda, row0, row_end, kb, la, wave, lane);
    issue_tile_rows<BN>(bmat, p.ldb, col0, p.N, kb, lb, wave, lane);
    issue_scales<BM>(p.sa, p.ldsa, row0, row_end, sbmat, nb0, NB - 1, KB, kb, ls, lw, wave,
                     lane);
  };

  auto compute = [&](const uint8_t* la, const uint8_t* lb, const float* ls, const float* lw) {
    const float sbv = lw[nb_local];
    v8i af[FM], bf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint8_t* rowp = la + (wm * WM + 16 * i + l16) * 128;
      const int4 lo = *reinterpret_cast<const int4*>(rowp + slot0 * 16);
      const int4 hi = *reinterpret_cast<const int4*>(rowp + slot1 * 16);
      af[i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint8_t* rowp = lb + (wn * WN + 16 * j + l16) * 128;
      const int4 lo = *reinterpret_cast<const int4*>(rowp + slot0 * 16);
      const int4 hi = *reinterpret_cast<const int4*>(rowp + slot1 * 16);
      bf[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    float4 sa4[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa4[i] = *reinterpret_cast<const float4*>(ls + wm * WM + 16 * i + 4 * g4);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const float w0 = sa4[i].x * sbv, w1 = sa4[i].y * sbv;
      const float w2 = sa4[i].z * sbv, w3 = sa4[i].w * sbv;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[i], bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
        acc[i][j][0] = __builtin_fmaf(part[0], w0, acc[i][j][0]);
        acc[i][j][1] = __builtin_fmaf(part[1], w1, acc[i][j][1]);
        acc[i][j][2] = __builtin_fmaf(part[2], w2, acc[i][j][2]);
        acc[i][j][3] = __builtin_fmaf(part[3], w3, acc[i][j][3]);
      }
    }
  };

  // Two LDS stages: while stage (kb & 1) feeds the MFMAs, group kb+1 streams
  // into the other one.  The wait + barrier at the top of each step makes the
  // stage just filled visible and retires all reads of the stage refilled next.
  issue(0, sA0, sB0, sS0, sW0);
  int64_t kb = 0;
  for (; kb + 1 < KB; kb += 2) {
    wait_vmem_all();
    __syncthreads();
    issue(kb + 1, sA1, sB1, sS1, sW1);
    compute(sA0, sB0, sS0, sW0);
    wait_vmem_all();
    __syncthreads();
    if (kb + 2 < KB) issue(kb + 2, sA0, sB0, sS0, sW0);
    compute(sA1, sB1, sS1, sW1);
  }
  if (kb < KB) {
    wait_vmem_all();
    __syncthreads();
    compute(sA0, sB0, sS0, sW0);
  }

  // Epilogue: lane holds rows 4*g4 + r, column l16 of each 16x16 tile.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = col0 + wn * WN + 16 * j + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + wm * WM + 16 * i + 4 * g4 + r;
        if (row < row_end && col < p.N) {
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

template <bool GROUPED>
hipError_t launch(const GemmArgs& args, bool out_bf16, hipStream_t stream) {
  constexpr int BM = 128, BN = 128;
  const int64_t NT = (args.N + BN - 1) / BN;
  const int64_t MT = GROUPED ? (args.M + BM - 1) / BM + args.G : (args.M + BM - 1) / BM;
  const int64_t blocks = MT * NT;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (out_bf16) {
    hipLaunchKernelGGL((block_gemm_kernel<BM, BN, GROUPED, true>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, args);
  } else {
    hipLaunchKernelGGL((block_gemm_kernel<BM, BN, GROUPED, false>), dim3((unsigned)blocks),
                       dim3(256), 0, stream, args);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_gemm(const GemmArgs& args, bool out_bf16, hipStream_t stream) {
  return launch<false>(args, out_bf16, stream);
}

hipError_t launch_grouped_gemm(const GemmArgs& args, bool out_bf16, hipStream_t stream) {
  return launch<true>(args, out_bf16, stream);
}

}  // namespace fp8bs
