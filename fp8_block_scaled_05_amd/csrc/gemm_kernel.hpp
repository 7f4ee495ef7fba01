// Block-scaled FP8 GEMM kernel template for gfx950 (dense and grouped/MoE).
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
// Structure: WM x WN waves per BM x BN output tile; each wave owns a
// (BM/WM) x (BN/WN) sub-tile made of 16x16 MFMA tiles.  Every K group of A
// and B is copied HBM->LDS by direct buffer_load ... lds (no register
// staging) into one of STAGES LDS buffers; the group's scales go through
// registers into a separate LDS array (with block-scaled B as the finished
// promotion factors S_A(row) * S_W(block), so that the MFMA loop does no
// arithmetic for them).  STAGES-1 groups are in flight while
// one feeds the MFMAs, and the copies of the next group are spread between
// the MFMA rows.  LDS rows are 128 bytes; the eight 16-byte chunks of a row
// are stored XOR-swizzled (lds_swizzle) so that the fragment reads are free
// of bank conflicts.  The lane K order inside an MFMA operand (32 bytes =
// chunks 2g, 2g+1 for lane group g) is the same for A and B, so products
// pair matching K.  Each MFMA's FP32 promotion is issued a few MFMAs later
// (a ring of partial products), so the VALU multiply-adds overlap the matrix
// cores.  B rows are staged permuted within each wave's columns so that a
// lane's MFMA columns are consecutive output columns (vector stores).
//
// Variants: fp32, bf16 or E4M3 output (the last quantized per 1x128 tile
// along N in the epilogue, the next GEMM's input); B scaled per 128x128
// block or, with RowScaledB, per row and K group (weight gradients); dense
// or grouped (MoE) tile schedules.
#pragma once

#include <atomic>

#include "device.hpp"
#include "internal.hpp"

namespace fp8bs {
namespace gemm {

typedef __attribute__((address_space(3))) void lds_void;

// LDS placement of the eight 16-byte K chunks of a 128-byte tile row: chunk c
// of row r is stored in slot c ^ lds_swizzle(r).  The function depends on
// r mod 16 only, so the MFMA reads (16 consecutive rows per fragment) can
// compute it from the lane index; with it the ds_read_b128 fragment reads of
// a wave are free of LDS bank conflicts on gfx950 (measured with
// SQ_LDS_BANK_CONFLICT; plain r & 7 or (r >> 1) & 7 leave 2-way conflicts).
__device__ __forceinline__ int lds_swizzle(int r) { return (r ^ ((r >> 3) & 1)) & 7; }

template <int BM_, int BN_, int WM_, int WN_, int STAGES_, int GROUP_M_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int STAGES = STAGES_, GROUP_M = GROUP_M_;
  static constexpr int NWAVES = WM * WN, THREADS = 64 * NWAVES;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  static constexpr int FM = TM / 16, FN = TN / 16;  // 16x16 MFMA tiles per wave
  // weight-block scales of the tile: one per 128 columns
  static constexpr int SB_COUNT = (BN + 127) / 128;
  // B scales per 128x128 block (false) or per row and K group (RowScaledB)
  static constexpr bool ROWB = false;
  // block-scaled B: the staged scales are the promotion factors
  // S_A(row) * S_W(block) for each of the tile's SB_COUNT weight blocks
  static constexpr bool PREMUL = true;
  // LDS stage: A rows | B rows; the scales of a stage live in a separate
  // array (activation scales, then weight-block scales) so that the compiler
  // can tell their register->LDS writes from the in-flight tile copies
  static constexpr int A_OFF = 0;
  static constexpr int B_OFF = BM * 128;
  static constexpr int STAGE_BYTES = B_OFF + BN * 128;
  // 1 KB (8 rows) per wave-wide direct load
  static constexpr int TILE_LOADS = (BM + BN) / 8 / NWAVES;
  // the scales go through registers and are written to LDS after the
  // compute, SREG items per thread per stage.  Block-scaled B: item
  // nb * BM + row is the factor S_A(row) * S_W(nb) of tile row `row` and the
  // tile's weight block nb, loaded as its two scales and multiplied before
  // the LDS write (spare items repeat the last block's factors)
  static constexpr int SCALE_ITEMS = SB_COUNT * BM;
  static constexpr int SREG = (SCALE_ITEMS + THREADS - 1) / THREADS;
  // every thread writes its SREG slots (no branch, so no merged wait counts)
  static constexpr int SCALE_FLOATS = SREG * THREADS;
  // vector-memory ops per wave per stage (two scale loads per item)
  static constexpr int LOADS = TILE_LOADS + 2 * SREG;
  static_assert((BM + BN) / 8 % NWAVES == 0, "tile loads must split evenly over waves");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave sub-tile must be whole MFMA tiles");
  static_assert(TN <= 128 && 128 % TN == 0, "a wave's columns must share one weight block");
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 LDS stages");
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget");
  static_assert(LOADS <= 63, "vmcnt range");
};

// The same tile configuration with B scaled per row and 128-K group (one
// scale per column of C per group, like the activation tiles of A) instead of
// per 128x128 block: the weight-gradient GEMM dW = dY^T . X, whose operands
// are both token-grouped activations.
template <class C>
struct RowScaledB : C {
  // items: the BM activation scales, then the BN row scales of B (the
  // factors differ per output element, so they are formed in the MFMA loop)
  static constexpr bool ROWB = true, PREMUL = false;
  static constexpr int SCALE_ITEMS = C::BM + C::BN;
  static constexpr int SREG = (SCALE_ITEMS + C::THREADS - 1) / C::THREADS;
  static constexpr int SCALE_FLOATS = SREG * C::THREADS;
  static constexpr int LOADS = C::TILE_LOADS + SREG;
  static_assert(LOADS <= 63, "vmcnt range");
};

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier after this wave's LDS writes (lgkmcnt) and all but its
// last N vector-memory ops have completed.  __syncthreads() would also wait
// for every direct-to-LDS copy still in flight (its release fence covers
// them), which would drain the copy pipeline at every K group; the memory
// clobber keeps the compiler from moving LDS accesses across the barrier.
template <int N>
__device__ __forceinline__ void barrier_after_vmcnt() {
  wait_vmcnt<N>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct TileCoords {
  int64_t row0, row_end, col0;
  const uint8_t* b;
  const float* sb;
  int64_t kb0, KB;  // the tile's K groups: kb0 .. kb0 + KB - 1 (KB >= 1)
  void* c;          // output matrix of the tile (row0, col0 relative to it)
};

// Tile schedules of one launch.
enum Sched {
  kDense = 0,     // one GEMM
  kGroupRows = 1, // row ranges of A per group, one B per group (MoE forward)
  kGroupK = 2     // K ranges per group, one C per group (MoE weight gradient)
};

// Workgroups are dealt round-robin to the 8 XCDs (workgroup b runs on XCD
// b mod 8): give each XCD a contiguous run of the raster of T tiles (the
// first T mod 8 XCDs one tile more than the others), so that concurrently
// resident tiles of one XCD share A and B in its L2.  A bijection of [0, T).
// Used where all tiles cost the same (dense); the grouped schedules, whose
// tiles differ in cost, keep the round-robin order instead.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t T) {
  const int64_t x = bid % 8, q = T / 8, r = T % 8;
  return x * q + (x < r ? x : r) + bid / 8;
}

// Coordinates of tile number `i` of a raster with MT tile-rows, which walks
// GROUP_M tile-rows before moving along N: tile-row tm, first column col0.
template <class C>
__device__ __forceinline__ void raster(const GemmArgs& p, int64_t i, int64_t MT, int64_t& tm,
                                       int64_t& col0) {
  const int64_t NT = (p.N + C::BN - 1) / C::BN;
  const int64_t per_group = (int64_t)C::GROUP_M * NT;
  const int64_t first_m = (i / per_group) * C::GROUP_M;
  const int64_t gsz = (MT - first_m) < C::GROUP_M ? (MT - first_m) : C::GROUP_M;
  const int64_t in_grp = i % per_group;
  tm = first_m + in_grp % gsz;
  col0 = (in_grp / gsz) * C::BN;
}

template <class C>
__device__ __forceinline__ void dense_tile(const GemmArgs& p, int64_t i, TileCoords& t) {
  int64_t tm;
  raster<C>(p, i, (p.M + C::BM - 1) / C::BM, tm, t.col0);
  t.b = p.b;
  t.sb = p.sb;
  t.row0 = tm * C::BM;
  t.row_end = p.M;
  t.kb0 = 0;
  t.KB = p.K / 128;
  t.c = p.c;
}

// Range [lo, hi) of group g from the device offsets, clamped to [0, limit]
// and to hi >= lo: offsets that break the documented contract then give
// unspecified results but no access outside the operands.
__device__ __forceinline__ void group_range(const GemmArgs& p, int64_t g, int64_t limit,
                                            int64_t& lo, int64_t& hi) {
  lo = p.group_offsets[g];
  hi = p.group_offsets[g + 1];
  lo = lo < 0 ? 0 : (lo > limit ? limit : lo);
  hi = hi < lo ? lo : (hi > limit ? limit : hi);
}

// Grouped along K: group g owns the K range [off[g], off[g+1]) (multiples of
// 128) and its own output C_g = c + g * c_group_stride; every group has the
// same MT x NT tiles, walked group after group.  KB == 0 for an empty group.
template <class C>
__device__ __forceinline__ void kgrouped_tile(const GemmArgs& p, int64_t i, TileCoords& t,
                                              int out_bytes) {
  const int64_t MT = (p.M + C::BM - 1) / C::BM;
  const int64_t per = MT * ((p.N + C::BN - 1) / C::BN);
  const int64_t g = i / per;
  int64_t tm;
  raster<C>(p, i % per, MT, tm, t.col0);
  t.b = p.b;
  t.sb = p.sb;
  t.row0 = tm * C::BM;
  t.row_end = p.M;
  int64_t o0, o1;
  group_range(p, g, p.K / 128 * 128, o0, o1);
  t.kb0 = o0 / 128;
  t.KB = o1 / 128 - t.kb0;
  t.c = static_cast<char*>(p.c) + g * p.c_group_stride * out_bytes;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, (unsigned)d, 64);
    v += lane >= d ? u : 0;
  }
  return v;
}

// Grouped raster: group g owns ceil(M_g / BM) tile-rows, in group order.
// The offsets are scanned 64 groups at a time by the whole wave (every wave
// of the workgroup computes the same, uniform, result).
template <class C>
__device__ __forceinline__ int group_row_tiles(const GemmArgs& p, int64_t g) {
  if (g >= p.G) return 0;
  int64_t lo, hi;
  group_range(p, g, p.M, lo, hi);
  return (int)((hi - lo + C::BM - 1) / C::BM);
}

// Total tile-rows over all groups.
template <class C>
__device__ __forceinline__ int64_t grouped_row_tiles(const GemmArgs& p) {
  const int lane = threadIdx.x & 63;
  int64_t total = 0;
  for (int64_t base = 0; base < p.G; base += 64)
    total += __builtin_amdgcn_readlane(wave_incl_sum(group_row_tiles<C>(p, base + lane)), 63);
  return total;
}

// Tile `i` of the grouped raster with MT (the total) tile-rows.
template <class C>
__device__ __forceinline__ void grouped_tile(const GemmArgs& p, int64_t i, int64_t MT,
                                             TileCoords& t) {
  const int64_t NB = (p.N + 127) / 128;
  const int lane = threadIdx.x & 63;
  int64_t tm;
  raster<C>(p, i, MT, tm, t.col0);
  // find the group holding tile-row tm (< MT, so the loop always finds it)
  int64_t seen = 0, g = 0, local = 0;
  for (int64_t base = 0; base < p.G; base += 64) {
    const int cnt = group_row_tiles<C>(p, base + lane);
    const int incl = wave_incl_sum(cnt);
    const int64_t chunk = __builtin_amdgcn_readlane(incl, 63);
    if (tm < seen + chunk) {
      const unsigned long long m = __ballot(seen + incl > tm);
      const int first = __builtin_ctzll(m);
      g = base + first;
      local = tm - seen - __builtin_amdgcn_readlane(incl - cnt, first);
      break;
    }
    seen += chunk;
  }
  int64_t lo, hi;
  group_range(p, g, p.M, lo, hi);
  t.row0 = lo + local * C::BM;
  t.row_end = hi;
  t.b = p.b + g * p.b_group_stride;
  t.sb = p.sb + g * NB * p.sb_ld;
  t.kb0 = 0;
  t.KB = p.K / 128;
  t.c = p.c;
}

// Loop-invariant per-lane byte offsets of one stage's direct copies,
// relative to wave-uniform bases (so each copy needs one 32-bit VGPR).
template <class C>
struct LoadPlan {
  uint32_t tile[C::TILE_LOADS];
  int32_t scale[C::SREG];  // element offset from the tile's S_A (or S_W) column base
  int32_t scaleb[C::SREG]; // factor items: element offset of the S_W block scale
};

// One stage's scales in registers: the S_A (or row-scaled S_W) value of each
// item, and with block-scaled B the item's S_W block scale.
template <class C>
struct ScaleRegs {
  float a[C::SREG];
  float b[C::PREMUL ? C::SREG : 1];
};

template <class C>
__device__ __forceinline__ void make_plan(const GemmArgs& p, const TileCoords& t, int wave,
                                          int lane, LoadPlan<C>& lp) {
  const int64_t NB = (p.N + 127) / 128;
  (void)wave;
  const int rows_a = (int)(t.row_end - t.row0);       // >= 1
  const int rows_b = (int)(p.N - t.col0);             // >= 1
#pragma unroll
  for (int j = 0; j < C::TILE_LOADS; ++j) {
    const int rbase = (wave * C::TILE_LOADS + j) * 8;  // first of 8 rows, A then B
    const int r = rbase + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swizzle(r);
    if (rbase < C::BM) {
      const int rr = r < rows_a ? r : rows_a - 1;
      lp.tile[j] = (uint32_t)rr * (uint32_t)p.lda + chunk * 16;
    } else {
      // B rows are staged permuted within each wave's TN columns: LDS row
      // 16 f + l of a wave's block holds tile column FN l + f, so the lane
      // that produces MFMA column l of fragment f holds, over f, FN
      // consecutive output columns (one vector store per output row)
      const int rb = r - C::BM, wb = rb / C::TN, rw = rb % C::TN;
      const int col = wb * C::TN + C::FN * (rw % 16) + rw / 16;
      const int rr = col < rows_b ? col : rows_b - 1;
      lp.tile[j] = (uint32_t)rr * (uint32_t)p.ldb + chunk * 16;
    }
  }
#pragma unroll
  for (int s = 0; s < C::SREG; ++s) {
    const int item = (int)threadIdx.x + s * C::THREADS;
    if constexpr (C::PREMUL) {
      // item = nb * BM + row: factor of tile row `row` and weight block nb
      // (blocks past the end of N, and spare items, repeat the last)
      const int row = item % C::BM;
      const int64_t nbl = NB - 1 - t.col0 / 128;
      int nb = item / C::BM;
      nb = nb < C::SB_COUNT ? nb : C::SB_COUNT - 1;
      lp.scale[s] = row < rows_a ? row : rows_a - 1;
      lp.scaleb[s] = (int)((nb < nbl ? nb : nbl) * p.sb_ld);
    } else if (item < C::BM) {
      lp.scale[s] = item < rows_a ? item : rows_a - 1;
    } else {
      // row-scaled B: row scale of tile column j (columns past N repeat the last)
      const int j = item - C::BM;
      lp.scale[s] = j < rows_b ? j : rows_b - 1;
    }
  }
}

// Buffer resources (base + byte range in SGPRs) of the tile's A rows, B rows,
// activation scales and weight-block scales.  Offsets never leave the range:
// rows past the edge are clamped to the last valid row.
struct Rsrc {
  __amdgpu_buffer_rsrc_t a, b;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  // raw (stride 0) buffer over [base, base + 4 GiB); 0x00020000 is the
  // gfx9 word-3 setting for untyped dword access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0xFFFFFFFF,
                                           0x00020000);
}

template <class C>
__device__ __forceinline__ Rsrc make_rsrc_set(const GemmArgs& p, const TileCoords& t) {
  Rsrc r;
  r.a = make_rsrc(p.a + t.row0 * p.lda + t.kb0 * 128);
  r.b = make_rsrc(t.b + t.col0 * p.ldb + t.kb0 * 128);
  return r;
}

// Issue tile copy number `idx` (0 <= idx < TILE_LOADS) of K group kb into one
// stage: a 1 KB block (8 rows x 128 B) of A, then of B.
template <class C>
__device__ __forceinline__ void issue_copy(const GemmArgs& p, const Rsrc& rs,
                                           const LoadPlan<C>& lp, int64_t kb, uint8_t* st,
                                           int wave, int idx) {
  (void)p;
  const int rbase = (wave * C::TILE_LOADS + idx) * 8;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rbase < C::BM ? rs.a : rs.b,
                                           (lds_void*)(st + rbase * 128), 16, lp.tile[idx],
                                           (int)(kb * 128), 0, 0);
}

// The scales of K group kb, one fp32 per item, into registers.  Issued before
// the group's tile copies, so that waiting for them (before they are written
// to LDS) leaves the tile copies in flight.
template <class C>
__device__ __forceinline__ void load_scales(const GemmArgs& p, const TileCoords& t,
                                            const LoadPlan<C>& lp, int64_t kb,
                                            ScaleRegs<C>& v) {
  const float* sa = p.sa + (t.kb0 + kb) * p.ldsa + t.row0;
  const float* sb = C::ROWB ? t.sb + (t.kb0 + kb) * p.sb_ld + t.col0
                            : t.sb + (t.col0 / 128) * p.sb_ld + t.kb0 + kb;
#pragma unroll
  for (int s = 0; s < C::SREG; ++s) {
    const int item = (int)threadIdx.x + s * C::THREADS;
    // one load instruction per item slot on every wave (uniform vmcnt counts)
    if constexpr (C::PREMUL) {
      (void)item;
      v.a[s] = sa[lp.scale[s]];
      v.b[s] = sb[lp.scaleb[s]];
    } else {
      const float* src = item < C::BM ? sa : sb;
      v.a[s] = src[lp.scale[s]];
    }
  }
}

template <class C>
__device__ __forceinline__ void store_scales(float* sc, const ScaleRegs<C>& v) {
#pragma unroll
  for (int s = 0; s < C::SREG; ++s)
    sc[(int)threadIdx.x + s * C::THREADS] = C::PREMUL ? v.a[s] * v.b[s] : v.a[s];
}

template <class C>
__device__ __forceinline__ void issue_stage(const GemmArgs& p, const Rsrc& rs,
                                            const LoadPlan<C>& lp, int64_t kb, uint8_t* st,
                                            int wave) {
#pragma unroll
  for (int idx = 0; idx < C::TILE_LOADS; ++idx) issue_copy<C>(p, rs, lp, kb, st, wave, idx);
}

typedef int v4i __attribute__((ext_vector_type(4)));

// Per-lane LDS byte offsets of a wave's MFMA operands inside a stage (the
// same for every stage).  They are made opaque to the optimizer once, so that
// each fragment address is the stage base plus one register plus a constant:
// the LDS lowering then tags every read with the stage's alias scope, and the
// wait-count pass can tell reads of a landed stage from copies still in
// flight to the other stages (an untagged read waits for every copy).
struct FragOffs {
  int a_lo, a_hi, b_lo, b_hi;  // K chunks 2g and 2g+1 of lane group g
  int sa;                      // float index of the lane's first row factor (block-scaled B:
                               // in its wave's weight block) or activation scale (row-scaled B)
  int sbc;                     // row-scaled B: float index of the lane's first column scale
};

template <class C>
__device__ __forceinline__ FragOffs frag_offsets(int wm, int wn, int lane) {
  const int l16 = lane & 15;
  // rows r (r mod 16 == l16) and the K chunk pair 2g, 2g+1 of lane group
  // g = lane / 16; chunk c of row r sits in slot c ^ lds_swizzle(r)
  const int slot0 = (2 * (lane >> 4)) ^ lds_swizzle(l16);
  FragOffs f;
  f.a_lo = C::A_OFF + (wm * C::TM + l16) * 128 + slot0 * 16;
  f.a_hi = C::A_OFF + (wm * C::TM + l16) * 128 + (slot0 ^ 1) * 16;
  f.b_lo = C::B_OFF + (wn * C::TN + l16) * 128 + slot0 * 16;
  f.b_hi = C::B_OFF + (wn * C::TN + l16) * 128 + (slot0 ^ 1) * 16;
  f.sa = wm * C::TM + 4 * (lane >> 4) + (C::PREMUL ? (wn * C::TN) / 128 * C::BM : 0);
  // the lane's FN output columns are consecutive (permuted B staging)
  f.sbc = C::BM + wn * C::TN + C::FN * l16;
  asm volatile("" : "+v"(f.a_lo), "+v"(f.a_hi), "+v"(f.b_lo), "+v"(f.b_hi), "+v"(f.sa));
  return f;
}

// Two 16-byte LDS reads -> one 32-byte MFMA operand (K chunks 2g, 2g+1).
__device__ __forceinline__ v8i load_frag(const uint8_t* st, int lo, int hi, int row_bytes) {
  const v4i a = *reinterpret_cast<const v4i*>(st + lo + row_bytes);
  const v4i b = *reinterpret_cast<const v4i*>(st + hi + row_bytes);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One K group from one LDS stage.  The wave's FM x FN MFMAs are issued in
// row-major order; the FP32 promotion of the MFMA issued RING steps earlier
// (long finished) follows each issue, so the VALU multiply-adds overlap the
// matrix cores.  The next stage's copies are spread between the MFMA rows (a
// burst of them would stall the wave at issue while the load pipe drains).
template <class C, bool REFILL, class Refill>
__device__ __forceinline__ void compute_stage(const uint8_t* st, const float* sc,
                                              const FragOffs& fo, v4f (&acc)[C::FM][C::FN],
                                              Refill&& issue_copy_n) {
  constexpr int NM = C::FM * C::FN;
  constexpr int RING = 4;
  // the promotion factors of row i are read until step i*FN + FN - 1 + RING
  // and their slot is refilled at step (i + WS)*FN
  constexpr int WS = 2 + (RING - 1) / C::FN;
  // With two stages the copies of the next group must land before this
  // step ends: issue them over the first half of the rows.  With more stages
  // they have a whole step of slack and are spread over all rows.
  constexpr int ISSUE_ROWS = C::STAGES == 2 ? (C::FM + 1) / 2 : C::FM;
  constexpr int PER_ROW = (C::TILE_LOADS + ISSUE_ROWS - 1) / ISSUE_ROWS;
  // block-scaled B: the stage holds the row factors of the wave's weight
  // block (fo.sa points into them); row-scaled B: the lane's FN column
  // scales, applied per MFMA tile
  static_assert(C::PREMUL != C::ROWB, "block-scaled B stages finished factors");
  float sbj[C::FN];
  if constexpr (C::ROWB) {
    if constexpr (C::FN % 4 == 0) {
#pragma unroll
      for (int q = 0; q < C::FN / 4; ++q) {
        const float4 v = *reinterpret_cast<const float4*>(sc + fo.sbc + 4 * q);
        sbj[4 * q] = v.x;
        sbj[4 * q + 1] = v.y;
        sbj[4 * q + 2] = v.z;
        sbj[4 * q + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int q = 0; q < C::FN; ++q) sbj[q] = sc[fo.sbc + q];
    }
  }
  // a lane's 4 rows of MFMA row i: one 16-byte LDS read (rows 16 i + 4 g .. + 3)
  const float* w4 = sc + fo.sa;
  v8i bf[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) bf[j] = load_frag(st, fo.b_lo, fo.b_hi, 16 * j * 128);
  v8i af[2];
  float4 s4[2];
  float w[WS][4];
  af[0] = load_frag(st, fo.a_lo, fo.a_hi, 0);
  s4[0] = *reinterpret_cast<const float4*>(w4);
  v4f ring[RING];
#pragma unroll
  for (int t = 0; t < NM + RING; ++t) {
    if (t >= RING) {
      const int u = t - RING, i = u / C::FN, j = u % C::FN;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = C::ROWB ? w[i % WS][r] * sbj[j] : w[i % WS][r];
        acc[i][j][r] = __builtin_fmaf(ring[u % RING][r], f, acc[i][j][r]);
      }
    }
    if (t < NM) {
      const int i = t / C::FN, j = t % C::FN;
      if (j == 0) {
        // this row's factors (S_A(row) * S_W, or S_A(row) with row-scaled B);
        // prefetch the next row
        w[i % WS][0] = s4[i & 1].x;
        w[i % WS][1] = s4[i & 1].y;
        w[i % WS][2] = s4[i & 1].z;
        w[i % WS][3] = s4[i & 1].w;
        if (i + 1 < C::FM) {
          af[(i + 1) & 1] = load_frag(st, fo.a_lo, fo.a_hi, 16 * (i + 1) * 128);
          s4[(i + 1) & 1] = *reinterpret_cast<const float4*>(w4 + 16 * (i + 1));
        }
      }
      ring[t % RING] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          af[i & 1], bf[j], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
      if (j == C::FN - 1 && REFILL) {
#pragma unroll
        for (int c = i * PER_ROW; c < (i + 1) * PER_ROW && c < C::TILE_LOADS; ++c) issue_copy_n(c);
      }
    }
    // One scheduling region per MFMA.  The partial products are separate
    // values, so without a fence the scheduler places each promotion right
    // after the MFMA that produces it (register pressure is lower there),
    // which stalls the wave on the MFMA latency (hazard NOPs); fenced, the
    // promotion stays RING MFMAs behind its producer.
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep this group's promotion inside this step: without a use here the
  // compiler sinks the multiply-adds past the next barrier, which piles two
  // groups' VALU work into one step.
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) asm volatile("" : "+v"(acc[i][j]));
}

// The LDS arrays of the kernel: one per pipeline stage for the tiles and one
// per stage for the scales (distinct objects, so that the compiler can tell
// the stages apart when it tracks copies in flight).
struct LdsSet {
  uint8_t* st[4];
  float* sc[4];
  float* red;  // E4M3 output: per-wave row maxima [WN][BM]
  float* rcp;  // E4M3 output: per-row reciprocals [BN/128][BM]
};

template <class T, int N>
struct Vec {
  typedef T type __attribute__((ext_vector_type(N)));
};

// The FN values of row r of MFMA row i held by one lane, as the output type:
// fp32, or bf16 packed two per dword (V_CVT_PK_BF16_F32, nearest even).
template <class C, int OUT>
struct RowVals {
  using T = typename std::conditional<OUT == kOutBF16, uint16_t, float>::type;
  typename Vec<T, C::FN>::type v;
  __device__ __forceinline__ RowVals(const v4f (&acc)[C::FM][C::FN], int i, int r) {
    if constexpr (OUT == kOutBF16 && C::FN % 2 == 0) {
      typename Vec<uint32_t, C::FN / 2>::type w;
#pragma unroll
      for (int q = 0; q < C::FN / 2; ++q) w[q] = bf16x2_rne(acc[i][2 * q][r], acc[i][2 * q + 1][r]);
      v = __builtin_bit_cast(typename Vec<T, C::FN>::type, w);
    } else {
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        if constexpr (OUT == kOutBF16) {
          v[j] = f32_to_bf16_rne(acc[i][j][r]);
        } else {
          v[j] = acc[i][j][r];
        }
      }
    }
  }
};

// fp32 or bf16 output.  Lane (g, l) holds rows 16 i + 4 g + r of the wave's
// sub-tile and, through the permuted B staging, the FN consecutive columns
// FN l .. FN l + FN - 1 of the wave's TN columns: one store per row (vector
// when the row start is aligned for it).  A wave whose whole sub-tile lies
// inside C (the common case) stores without per-row tests.
template <class C, int OUT>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const TileCoords& t,
                                           const v4f (&acc)[C::FM][C::FN], int wm, int wn,
                                           int lane) {
  using T = typename RowVals<C, OUT>::T;
  using VT = typename Vec<T, C::FN>::type;
  const int g4 = lane >> 4, l16 = lane & 15;
  const int64_t col = t.col0 + wn * C::TN + C::FN * l16;
  const bool vec = C::FN > 1 && reinterpret_cast<uintptr_t>(t.c) % (C::FN * sizeof(T)) == 0 &&
                   p.ldc % C::FN == 0;
  T* const out = reinterpret_cast<T*>(t.c);
  const int64_t wrow0 = t.row0 + wm * C::TM;
  // wave-uniform: every row and column of the wave's sub-tile is inside C
  const bool inside = vec && wrow0 + C::TM <= t.row_end && t.col0 + (wn + 1) * C::TN <= p.N;
  if constexpr (C::FN > 1) {
    if (inside) {
      T* const base = out + (wrow0 + 4 * g4) * p.ldc + col;
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const RowVals<C, OUT> rv(acc, i, r);
          *reinterpret_cast<VT*>(base + (16 * i + r) * p.ldc) = rv.v;
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = wrow0 + 16 * i + 4 * g4 + r;
      if (row >= t.row_end) continue;
      const RowVals<C, OUT> rv(acc, i, r);
      T* const dst = out + row * p.ldc + col;
      if constexpr (C::FN > 1) {
        if (vec && col + C::FN <= p.N) {
          *reinterpret_cast<VT*>(dst) = rv.v;
          continue;
        }
      }
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        if (col + j < p.N) dst[j] = rv.v[j];
    }
  }
}

// E4M3 output quantized per 1x128 tile along N, the next layer's FP8 input
// (pages: "How online quantization in DeepSeek-V3 differs from delayed
// quantization", item 1, and "How the unified E4M3 format adds to
// DeepSeek-V3's efficiency", section "Fine-grained quantization strategy":
// the same online 1x128 activation quantization, applied to the FP32 output
// before it leaves the kernel).  A row's 128-column tile spans 128 / TN
// waves: each wave reduces its TN columns (lanes, then the 16 lanes of a
// DPP row), the partial maxima meet in LDS, one thread per (row, tile)
// forms the scale and reciprocal exactly as the activation quantizer does,
// and each lane converts and stores its FN consecutive codes per row.
// Requires BN % 128 == 0 and N % 128 == 0 (whole tiles).
template <class C>
__device__ __forceinline__ void store_tile_e4m3(const GemmArgs& p, const TileCoords& t,
                                                const v4f (&acc)[C::FM][C::FN], int wm,
                                                int wn, int lane, float* red, float* rcp) {
  static_assert(C::BN % 128 == 0, "E4M3 output needs whole 128-column tiles per workgroup");
  constexpr int WPB = 128 / C::TN;  // waves across one 128-column tile
  constexpr int NBT = C::BN / 128;  // 128-column tiles per workgroup tile
  const int g4 = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) m = fmaxf(m, fabsf(acc[i][j][r]));
      m = max_row16(m);
      if (l16 == 0) red[wn * C::BM + wm * C::TM + 16 * i + 4 * g4 + r] = m;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < NBT * C::BM; idx += C::THREADS) {
    const int nb = idx / C::BM, rt = idx % C::BM;
    float amax = 0.f;
#pragma unroll
    for (int w = 0; w < WPB; ++w) amax = fmaxf(amax, red[(nb * WPB + w) * C::BM + rt]);
    float s, rr;
    group_scale(amax, s, rr);
    rcp[idx] = rr;
    const int64_t row = t.row0 + rt, cb = t.col0 / 128 + nb;
    if (row < t.row_end && cb * 128 < p.N) p.sc[cb * p.ldsc + row] = s;
  }
  __syncthreads();
  const int64_t col = t.col0 + wn * C::TN + C::FN * l16;
  if (col >= p.N) return;  // the wave's whole 128-column tile is past N
  const int nbw = (wn * C::TN) / 128;
  uint8_t* const out = reinterpret_cast<uint8_t*>(t.c);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const float4 r4 =
        *reinterpret_cast<const float4*>(rcp + nbw * C::BM + wm * C::TM + 16 * i + 4 * g4);
    const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = t.row0 + wm * C::TM + 16 * i + 4 * g4 + r;
      if (row >= t.row_end) continue;
      uint8_t* const dst = out + row * p.ldc + col;
      float y[C::FN];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) y[j] = acc[i][j][r] * rv[r];
      if constexpr (C::FN == 1) {
        *dst = (uint8_t)cvt2_e4m3<false>(y[0], 0.f, 0u);
      } else if constexpr (C::FN == 2) {
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)cvt2_e4m3<false>(y[0], y[1], 0u);
      } else {
        static_assert(C::FN % 4 == 0, "FN of 1, 2 or a multiple of 4");
        typename Vec<uint32_t, C::FN / 4>::type w;
#pragma unroll
        for (int q = 0; q < C::FN / 4; ++q) {
          const uint32_t lo = cvt2_e4m3<false>(y[4 * q], y[4 * q + 1], 0u);
          w[q] = cvt2_e4m3<true>(y[4 * q + 2], y[4 * q + 3], lo);
        }
        *reinterpret_cast<typename Vec<uint32_t, C::FN / 4>::type*>(dst) = w;
      }
    }
  }
}

template <class C, int OUT>
__device__ __forceinline__ void block_gemm_body(const GemmArgs& p, const TileCoords& t,
                                                const LdsSet& L) {
  // wave index in an SGPR so that per-wave values stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int64_t KB = t.KB;

  LoadPlan<C> lp;
  make_plan<C>(p, t, wave, lane, lp);
  const FragOffs fo = frag_offsets<C>(wm, wn, lane);
  const Rsrc rs = make_rsrc_set<C>(p, t);

  v4f acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Pipeline: group g lives in LDS stage g % STAGES.  Step kb waits for this
  // wave's copies of group kb (leaving the copies of later groups in flight),
  // meets the other waves at a barrier (so every copy of group kb is visible
  // and every wave has finished reading the stage about to be refilled),
  // refills that stage with group kb + STAGES - 1, then computes group kb.
  // The steady-state loop always refills; the last steps are peeled.
  auto stg = [&](int i) -> uint8_t* { return L.st[i]; };
  auto scl = [&](int i) -> float* { return L.sc[i]; };
  // Group g lives in stage g % STAGES.  The scales of group g are loaded to
  // registers with its tile copies (at step g - STAGES + 1) but written to
  // the stage's scale array only at the end of step g - 1: a register ring of
  // SLEAD = STAGES - 2 scale sets gives their loads the same slack as the
  // tile copies (without it, short steps wait for the scale loads).
  // Every prologue stage is filled (with the last group again when KB is
  // smaller than STAGES - 1; such a stage is never read): a conditional fill
  // would make the compiler assume, at the top of the steady loop, that
  // stage 0 may still be in flight.  The extra copies are issued after every
  // real group, so the drain's waits (which count real groups only) still
  // cover them.
  constexpr int SLEAD = C::STAGES - 2;
  ScaleRegs<C> carry[SLEAD > 0 ? SLEAD : 1];
#pragma unroll
  for (int s = 0; s < C::STAGES - 1; ++s) {
    const int64_t g = s < KB ? s : KB - 1;
    ScaleRegs<C> sv;
    load_scales<C>(p, t, lp, g, sv);
    issue_stage<C>(p, rs, lp, g, stg(s), wave);
    if (s == 0) {
      store_scales<C>(scl(0), sv);
    } else {
      carry[s - 1] = sv;
    }
  }
  // end of the step of group k (stage index u = k % STAGES): write the scales
  // of group k + 1, then shift the ring (cur: the scales loaded this step,
  // group k + STAGES - 1)
  auto retire_scales = [&](int u, const ScaleRegs<C>& cur, bool store_next) {
    if constexpr (SLEAD == 0) {
      if (store_next) store_scales<C>(scl((u + 1) % C::STAGES), cur);
    } else {
      if (store_next) store_scales<C>(scl((u + 1) % C::STAGES), carry[0]);
#pragma unroll
      for (int d = 0; d + 1 < SLEAD; ++d) carry[d] = carry[d + 1];
      carry[SLEAD - 1] = cur;
    }
  };

  // wait until at most `later` groups (issued after group kb) are in flight
  auto wait_and_sync = [&](int later) {
    if (C::STAGES > 3 && later >= 2) {
      barrier_after_vmcnt<C::LOADS * (C::STAGES > 3 ? 2 : 0)>();
    } else if (C::STAGES > 2 && later >= 1) {
      barrier_after_vmcnt<C::LOADS * (C::STAGES > 2 ? 1 : 0)>();
    } else {
      barrier_after_vmcnt<0>();
    }
  };

  int64_t kb = 0;
  // steady state: STAGES steps per iteration, each refilling the stage read
  // in the previous step with copies interleaved into its MFMA stream
  for (; kb + 2 * C::STAGES - 2 < KB; kb += C::STAGES) {
#pragma unroll
    for (int u = 0; u < C::STAGES; ++u) {
      wait_and_sync(C::STAGES - 2);
      uint8_t* const nxt = stg((u + C::STAGES - 1) % C::STAGES);
      const int64_t kn = kb + u + C::STAGES - 1;
      ScaleRegs<C> sv;
      load_scales<C>(p, t, lp, kn, sv);
      // keep the scale loads ahead of this step's tile copies (in-order
      // completion then lets their wait leave the tile copies in flight)
      __builtin_amdgcn_sched_barrier(0);
      compute_stage<C, true>(stg(u), scl(u), fo, acc, [&](int c) {
        issue_copy<C>(p, rs, lp, kn, nxt, wave, c);
      });
      retire_scales(u, sv, true);
    }
  }
  // drain: at most 2*STAGES-2 steps remain; unrolled so stage indices stay
  // compile-time constants; any refill is issued before the compute
#pragma unroll
  for (int u = 0; u < 2 * C::STAGES - 2; ++u) {
    const int64_t k = kb + u;
    if (k < KB) {
      const int64_t last = k + C::STAGES - 2 < KB - 1 ? k + C::STAGES - 2 : KB - 1;
      wait_and_sync((int)(last - k));
      uint8_t* const nxt = stg((u + C::STAGES - 1) % C::STAGES);
      const bool refill = k + C::STAGES - 1 < KB;
      ScaleRegs<C> sv{};
      if (refill) {
        load_scales<C>(p, t, lp, k + C::STAGES - 1, sv);
        issue_stage<C>(p, rs, lp, k + C::STAGES - 1, nxt, wave);
      }
      compute_stage<C, false>(stg(u % C::STAGES), scl(u % C::STAGES), fo, acc, [](int) {});
      retire_scales(u % C::STAGES, sv, SLEAD == 0 ? refill : k + 1 < KB);
    }
  }

  if constexpr (OUT == kOutE4M3) {
    store_tile_e4m3<C>(p, t, acc, wm, wn, lane, L.red, L.rcp);
  } else {
    store_tile<C, OUT>(p, t, acc, wm, wn, lane);
  }
}

// A tile of a group without K range: C_g = 0 there (fp32 or bf16 output).
template <class C, int OUT>
__device__ __forceinline__ void store_zero_tile(const GemmArgs& p, const TileCoords& t) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  v4f zero[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) zero[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  store_tile<C, OUT>(p, t, zero, wave / C::WN, wave % C::WN, threadIdx.x & 63);
}

// One launch covers the raster of BM x BN tiles.
// Dense and grouped-along-K: when the raster would end in a partial round of
// at most half the compute units' worth of tiles, those last tiles are split
// into two TAIL (half-height) tiles each, so the last round takes half as
// long: workgroups [0, full) take whole tiles, the rest take half tiles.
// Grouped rows: the grid is an upper bound on the tile count (the group
// sizes live on the device); the workgroups past the real count exit at
// once, and a group's last tile-row runs as a TAIL tile when it holds at
// most TAIL::BM rows.  TAIL == C: no half tiles.
// The buffer-resource type exists only for the device; the host pass sees an
// empty kernel (it only needs the launch stub).
template <class C, class TAIL, int SCHED, int OUT>
__global__ __launch_bounds__(C::THREADS) void block_gemm_kernel(GemmArgs p, int64_t full) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert((TAIL::THREADS == C::THREADS && TAIL::BN == C::BN && 2 * TAIL::BM == C::BM) ||
                    std::is_same<C, TAIL>::value, "tail tiles are half-height tiles");
  static_assert(SCHED != kGroupK || OUT != kOutE4M3, "grouped-K output is fp32 or bf16");
  constexpr int SB = C::STAGE_BYTES > TAIL::STAGE_BYTES ? C::STAGE_BYTES : TAIL::STAGE_BYTES;
  constexpr int SF = C::SCALE_FLOATS > TAIL::SCALE_FLOATS ? C::SCALE_FLOATS : TAIL::SCALE_FLOATS;
  constexpr int NS = C::STAGES > TAIL::STAGES ? C::STAGES : TAIL::STAGES;
  constexpr bool HALVES = !std::is_same<C, TAIL>::value;
  __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
  __shared__ __attribute__((aligned(16))) uint8_t st2[NS > 2 ? SB : 16];
  __shared__ __attribute__((aligned(16))) uint8_t st3[NS > 3 ? SB : 16];
  __shared__ __attribute__((aligned(16))) float sc0[SF];
  __shared__ __attribute__((aligned(16))) float sc1[SF];
  __shared__ __attribute__((aligned(16))) float sc2[NS > 2 ? SF : 4];
  __shared__ __attribute__((aligned(16))) float sc3[NS > 3 ? SF : 4];
  constexpr bool Q = OUT == kOutE4M3;
  __shared__ __attribute__((aligned(16))) float red[Q ? C::WN * C::BM : 4];
  __shared__ __attribute__((aligned(16))) float rcp[Q ? C::BN / 128 * C::BM : 4];
  const LdsSet L{{st0, st1, st2, st3}, {sc0, sc1, sc2, sc3}, red, rcp};
  const int64_t bid = blockIdx.x;
  TileCoords t;
  if constexpr (SCHED == kGroupRows) {
    (void)full;
    const int64_t MT = grouped_row_tiles<C>(p);
    const int64_t T = MT * ((p.N + C::BN - 1) / C::BN);
    if (bid >= T) return;  // whole workgroup: past the last real tile
    // tiles dealt round-robin over the XCDs (not in contiguous runs): the
    // groups' short last tile-rows and the raster's end then spread evenly
    grouped_tile<C>(p, bid, MT, t);
    if constexpr (HALVES) {
      if (t.row_end - t.row0 <= TAIL::BM) {
        block_gemm_body<TAIL, OUT>(p, t, L);
        return;
      }
    }
    block_gemm_body<C, OUT>(p, t, L);
  } else {
    constexpr int out_bytes = OUT == kOutF32 ? 4 : OUT == kOutBF16 ? 2 : 1;
    auto tile_of = [&](int64_t i) {
      if constexpr (SCHED == kGroupK) {
        kgrouped_tile<C>(p, i, t, out_bytes);
      } else {
        dense_tile<C>(p, i, t);
      }
    };
    // grouped along K: the groups' K lengths differ, so contiguous runs per
    // XCD (equal tile counts) would give the XCDs unequal work; dealing
    // the tiles round-robin gives every XCD tiles of every group
    auto order = [&](int64_t i, int64_t n) {
      return SCHED == kGroupK ? i : xcd_remap(i, n);
    };
    if (bid < full) {
      tile_of(order(bid, full));
      if constexpr (SCHED == kGroupK) {
        if (t.KB == 0) {  // whole workgroup: a group without K range
          store_zero_tile<C, OUT>(p, t);
          return;
        }
      }
      block_gemm_body<C, OUT>(p, t, L);
    } else if constexpr (HALVES) {
      const int64_t j = order(bid - full, (int64_t)gridDim.x - full);
      tile_of(full + j / 2);
      t.row0 += (j & 1) * TAIL::BM;
      if (t.row0 >= t.row_end) return;  // lower half below the last row
      if constexpr (SCHED == kGroupK) {
        if (t.KB == 0) {
          store_zero_tile<TAIL, OUT>(p, t);
          return;
        }
      }
      block_gemm_body<TAIL, OUT>(p, t, L);
    }
  }
#endif
}

// Compute units of the current device, cached per device.  Any thread may
// fill an entry; racing fills store the same value, and the relaxed atomics
// make the race well defined.
inline int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class C, int SCHED, class TAIL = C>
hipError_t launch(const GemmArgs& args, OutKind out, hipStream_t stream) {
  const int64_t NT = (args.N + C::BN - 1) / C::BN;
  int64_t MT = (args.M + C::BM - 1) / C::BM;
  // grouped rows: every non-empty group adds at most one partial tile-row,
  // and every tile-row holds at least one row
  if (SCHED == kGroupRows) MT = MT + args.G < args.M ? MT + args.G : args.M;
  // grouped K: the same tiles for every group
  const int64_t tiles = MT * NT * (SCHED == kGroupK ? args.G : 1);
  if (tiles <= 0) return hipSuccess;
  int64_t full = tiles, blocks = tiles;
  if (SCHED != kGroupRows && !std::is_same<C, TAIL>::value) {
    // split the last partial round only when its halves fit in one round
    // (at most half the compute units' worth of tiles): a larger tail would
    // take 1.5 rounds of half tiles, longer than one round of whole tiles
    const int64_t cus = device_cus();
    const int64_t tail = cus > 0 ? tiles % cus : 0;
    if (cus > 0 && tiles > cus && tail != 0 && 2 * tail <= cus) {
      full = tiles - tail;
      blocks = full + 2 * tail;
    }
  }
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(C::THREADS);
  switch (out) {
    case kOutF32:
      return launch_kernel(block_gemm_kernel<C, TAIL, SCHED, kOutF32>, grid, block, stream, args,
                           full);
    case kOutBF16:
      return launch_kernel(block_gemm_kernel<C, TAIL, SCHED, kOutBF16>, grid, block, stream,
                           args, full);
    default:
      if constexpr (C::BN % 128 == 0 && !C::ROWB && SCHED != kGroupK) {
        return launch_kernel(block_gemm_kernel<C, TAIL, SCHED, kOutE4M3>, grid, block, stream,
                             args, full);
      } else {
        // E4M3 output needs whole 128-column tiles; row-scaled B (weight
        // gradients) has fp32 and bf16 outputs only
        return hipErrorInvalidConfiguration;
      }
  }
}

}  // namespace gemm
}  // namespace fp8bs
