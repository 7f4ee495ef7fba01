// C ABI of libfp8bs: argument validation (before any HIP call) and dispatch
// to the gfx950 kernels.  Declarations and the contract are in
// include/fp8bs.h.

#include <atomic>

#include "fp8bs.h"
#include "internal.hpp"

// Device buffer of fp8_block_gemm_bf16_noalloc: the E4M3 codes and scales of
// A quantized inside the call.  Each GPU that loads the library holds its own
// copy until the process ends.  Host code never uses this name as a device
// address (on the host it only names the variable); it uses the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[FP8BS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kTile = 128;
constexpr int64_t kMaxGroups = 4096;
constexpr int64_t kMaxHistory = 4096;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool ld_ok(int64_t ld, int64_t row) { return ld >= row && ld % 16 == 0; }

// GEMM operands: the tile copies address up to 256 rows from the tile's
// first row with 32-bit byte offsets (row * ld + k)
constexpr int64_t kMaxOperandLd = int64_t(1) << 24;
bool operand_ld_ok(int64_t ld, int64_t row) { return ld_ok(ld, row) && ld <= kMaxOperandLd; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FP8BS_OK;
  g_last_hip_error = static_cast<int>(e);
  return FP8BS_ERR_HIP;
}

size_t fused_q_bytes(int64_t M, int64_t K) { return round256(size_t(M) * size_t(K)); }
size_t fused_s_bytes(int64_t M, int64_t K) { return round256(size_t(K / kTile) * size_t(M) * 4); }

}  // namespace

extern "C" {

int fp8_quant_act_1x128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                        int64_t ldq, float* s, int64_t lds, void* stream) {
  if (M < 0 || K <= 0 || K % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M == 0) return FP8BS_OK;
  if (!x || !q || !s) return FP8BS_ERR_NULL;
  if (!ld_ok(ldx, K) || !ld_ok(ldq, K) || lds < M) return FP8BS_ERR_LAYOUT;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8BS_ERR_LAYOUT;
  return hip_status(fp8bs::launch_quant_act(x, M, K, ldx, q, ldq, s, lds,
                                            static_cast<hipStream_t>(stream)));
}

int fp8_quant_act_1x128_delayed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds, int mode,
                                float* hist, int64_t ldh, int64_t H, int64_t step,
                                uint32_t* stats, void* stream) {
  if (mode != FP8BS_DELAY_TILE && mode != FP8BS_DELAY_TENSOR) return FP8BS_ERR_DTYPE;
  if (M < 0 || K <= 0 || K % kTile != 0 || H < 1 || H > kMaxHistory || step < 0)
    return FP8BS_ERR_SHAPE;
  if (M == 0) return FP8BS_OK;
  if (!x || !q || !s || !hist) return FP8BS_ERR_NULL;
  if (!ld_ok(ldx, K) || !ld_ok(ldq, K) || lds < M) return FP8BS_ERR_LAYOUT;
  if (mode == FP8BS_DELAY_TILE && ldh < M) return FP8BS_ERR_LAYOUT;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(hist, 4) ||
      (stats && !aligned(stats, 4)))
    return FP8BS_ERR_LAYOUT;
  return hip_status(fp8bs::launch_quant_act_delayed(x, M, K, ldx, q, ldq, s, lds,
                                                    mode == FP8BS_DELAY_TENSOR, hist, ldh, H,
                                                    step, stats,
                                                    static_cast<hipStream_t>(stream)));
}

int fp8_quant_w_128x128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                        int64_t ldq, float* s, void* stream) {
  if (N < 0 || K <= 0 || K % kTile != 0) return FP8BS_ERR_SHAPE;
  if (N == 0) return FP8BS_OK;
  if (!w || !q || !s) return FP8BS_ERR_NULL;
  if (!ld_ok(ldw, K) || !ld_ok(ldq, K)) return FP8BS_ERR_LAYOUT;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4)) return FP8BS_ERR_LAYOUT;
  return hip_status(fp8bs::launch_quant_w(w, N, K, ldw, q, ldq, s, nullptr, 0, nullptr,
                                          static_cast<hipStream_t>(stream)));
}

int fp8_quant_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, uint8_t* q,
                     int64_t ldq, float* s, int64_t lds, const uint16_t* w, int64_t N,
                     int64_t ldw, uint8_t* qw, int64_t ldqw, float* sw, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || K % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 && N == 0) return FP8BS_OK;
  if (M > 0 && (!x || !q || !s)) return FP8BS_ERR_NULL;
  if (N > 0 && (!w || !qw || !sw)) return FP8BS_ERR_NULL;
  if (M > 0 && (!ld_ok(ldx, K) || !ld_ok(ldq, K) || lds < M || !aligned(x, 16) ||
                !aligned(q, 16) || !aligned(s, 4)))
    return FP8BS_ERR_LAYOUT;
  if (N > 0 && (!ld_ok(ldw, K) || !ld_ok(ldqw, K) || !aligned(w, 16) || !aligned(qw, 16) ||
                !aligned(sw, 4)))
    return FP8BS_ERR_LAYOUT;
  return hip_status(fp8bs::launch_quant_linear(x, M, K, ldx, q, ldq, s, lds, w, N, ldw, qw,
                                               ldqw, sw, static_cast<hipStream_t>(stream)));
}

int fp8_quant_act_128x1_t(const uint16_t* x, int64_t M, int64_t N, int64_t ldx, uint8_t* qt,
                          int64_t ldqt, float* st, int64_t ldst, void* stream) {
  if (M < 0 || N < 0 || M % kTile != 0 || N % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!x || !qt || !st) return FP8BS_ERR_NULL;
  if (!ld_ok(ldx, N) || !ld_ok(ldqt, M) || ldst < N) return FP8BS_ERR_LAYOUT;
  if (!aligned(x, 16) || !aligned(qt, 16) || !aligned(st, 4)) return FP8BS_ERR_LAYOUT;
  return hip_status(fp8bs::launch_quant_act_128x1_t(x, M, N, ldx, qt, ldqt, st, ldst,
                                                    static_cast<hipStream_t>(stream)));
}

int fp8_quant_w_128x128_t(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                          int64_t ldq, float* s, uint8_t* qt, int64_t ldqt, float* st,
                          void* stream) {
  if (N < 0 || K <= 0 || K % kTile != 0 || N % kTile != 0) return FP8BS_ERR_SHAPE;
  if (N == 0) return FP8BS_OK;
  if (!w || !q || !s || !qt || !st) return FP8BS_ERR_NULL;
  if (!ld_ok(ldw, K) || !ld_ok(ldq, K) || !ld_ok(ldqt, N)) return FP8BS_ERR_LAYOUT;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(qt, 16) ||
      !aligned(st, 4))
    return FP8BS_ERR_LAYOUT;
  return hip_status(fp8bs::launch_quant_w(w, N, K, ldw, q, ldq, s, qt, ldqt, st,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared body of the dense entry points.  out: element type of c; for E4M3
// output, sc/ldsc receive the per-1x128 output scales.
int block_gemm_impl(int a_kind, const void* a, int64_t lda, float* sa, int64_t ldsa,
                    const uint8_t* b, int64_t ldb, const float* sb, void* c, int64_t ldc,
                    fp8bs::OutKind out, float* sc, int64_t ldsc, int64_t M, int64_t N,
                    int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  if (a_kind != FP8BS_A_E4M3 && a_kind != FP8BS_A_BF16) return FP8BS_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || K % kTile != 0) return FP8BS_ERR_SHAPE;
  if (out == fp8bs::kOutE4M3 && N % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!a || !b || !sb || !c) return FP8BS_ERR_NULL;
  if (a_kind == FP8BS_A_E4M3 && !sa) return FP8BS_ERR_NULL;
  if (out == fp8bs::kOutE4M3 && !sc) return FP8BS_ERR_NULL;
  if (!operand_ld_ok(lda, K) || !operand_ld_ok(ldb, K) || ldc < N) return FP8BS_ERR_LAYOUT;
  if (sa && ldsa < M) return FP8BS_ERR_LAYOUT;
  const uintptr_t c_align = out == fp8bs::kOutF32 ? 4 : out == fp8bs::kOutBF16 ? 2 : 16;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, c_align) || !aligned(sb, 4) ||
      (sa && !aligned(sa, 4)))
    return FP8BS_ERR_LAYOUT;
  if (out == fp8bs::kOutE4M3 && (!ld_ok(ldc, N) || ldsc < M || !aligned(sc, 4)))
    return FP8BS_ERR_LAYOUT;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf16_a = a_kind == FP8BS_A_BF16;
  if (bf16_a) {
    // the caller's workspace is required for every bf16-A call (the
    // few-row path below does not use it)
    const size_t need = fp8bs_workspace_bytes(FP8BS_OP_GEMM_BF16, M, N, K, 0);
    if (!workspace || workspace_bytes < need) return FP8BS_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return FP8BS_ERR_LAYOUT;
  }
  if (bf16_a && M <= fp8bs::kFewRowsFused && out != fp8bs::kOutE4M3) {
    // very few rows: the weight-stream kernel quantizes A itself
    return hip_status(fp8bs::launch_few_rows_gemm(a, lda, sa, ldsa, true, b, ldb, sb, c, ldc,
                                                  out == fp8bs::kOutBF16, M, N, K, st));
  }

  fp8bs::GemmArgs g{};
  g.b = b;
  g.ldb = ldb;
  g.sb = sb;
  g.c = c;
  g.ldc = ldc;
  g.sc = sc;
  g.ldsc = ldsc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.sb_ld = K / kTile;
  if (a_kind == FP8BS_A_E4M3) {
    g.a = static_cast<const uint8_t*>(a);
    g.lda = lda;
    g.sa = sa;
    g.ldsa = ldsa;
  } else {
    uint8_t* wq = static_cast<uint8_t*>(workspace);
    float* ws = sa ? sa : reinterpret_cast<float*>(wq + fused_q_bytes(M, K));
    const int64_t wlds = sa ? ldsa : M;
    int st0 = hip_status(fp8bs::launch_quant_act(static_cast<const uint16_t*>(a), M, K, lda, wq,
                                                 K, ws, wlds, st));
    if (st0 != FP8BS_OK) return st0;
    g.a = wq;
    g.lda = K;
    g.sa = ws;
    g.ldsa = wlds;
  }
  if (M <= fp8bs::kFewRows && out != fp8bs::kOutE4M3)
    return hip_status(fp8bs::launch_few_rows_gemm(g.a, g.lda, const_cast<float*>(g.sa), g.ldsa,
                                                  false, b, ldb, sb, c, ldc,
                                                  out == fp8bs::kOutBF16, M, N, K, st));
  return hip_status(fp8bs::launch_block_gemm(g, out, st));
}

// Shared body of the grouped entry points.
int grouped_gemm_impl(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                      const uint8_t* b, int64_t ldb, int64_t b_group_stride, const float* sb,
                      void* c, int64_t ldc, fp8bs::OutKind out, float* sc, int64_t ldsc,
                      const int32_t* group_offsets, int64_t G, int64_t M_total, int64_t N,
                      int64_t K, void* stream) {
  if (G < 1 || G > kMaxGroups || M_total < 0 || N < 0 || K <= 0 || K % kTile != 0)
    return FP8BS_ERR_SHAPE;
  if (out == fp8bs::kOutE4M3 && N % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M_total == 0 || N == 0) return FP8BS_OK;
  if (!a || !sa || !b || !sb || !c || !group_offsets) return FP8BS_ERR_NULL;
  if (out == fp8bs::kOutE4M3 && !sc) return FP8BS_ERR_NULL;
  if (!operand_ld_ok(lda, K) || !operand_ld_ok(ldb, K) || ldc < N || ldsa < M_total)
    return FP8BS_ERR_LAYOUT;
  if (b_group_stride % 16 != 0 || b_group_stride < (N - 1) * ldb + K) return FP8BS_ERR_LAYOUT;
  const uintptr_t c_align = out == fp8bs::kOutF32 ? 4 : out == fp8bs::kOutBF16 ? 2 : 16;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, c_align) || !aligned(sa, 4) ||
      !aligned(sb, 4) || !aligned(group_offsets, 4))
    return FP8BS_ERR_LAYOUT;
  if (out == fp8bs::kOutE4M3 && (!ld_ok(ldc, N) || ldsc < M_total || !aligned(sc, 4)))
    return FP8BS_ERR_LAYOUT;
  fp8bs::GemmArgs g{};
  g.a = a;
  g.lda = lda;
  g.sa = sa;
  g.ldsa = ldsa;
  g.b = b;
  g.ldb = ldb;
  g.b_group_stride = b_group_stride;
  g.sb = sb;
  g.c = c;
  g.ldc = ldc;
  g.sc = sc;
  g.ldsc = ldsc;
  g.M = M_total;
  g.N = N;
  g.K = K;
  g.sb_ld = K / kTile;
  g.group_offsets = group_offsets;
  g.G = G;
  return hip_status(fp8bs::launch_grouped_gemm(g, out, static_cast<hipStream_t>(stream)));
}

fp8bs::OutKind out_of(int out_kind) {
  return out_kind == FP8BS_OUT_BF16 ? fp8bs::kOutBF16 : fp8bs::kOutF32;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.  Concurrent first calls on one
// device store the same address.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

int fp8_block_gemm(int a_kind, const void* a, int64_t lda, float* sa, int64_t ldsa,
                   const uint8_t* b, int64_t ldb, const float* sb, void* c, int64_t ldc,
                   int out_kind, int64_t M, int64_t N, int64_t K, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (out_kind != FP8BS_OUT_F32 && out_kind != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
  return block_gemm_impl(a_kind, a, lda, sa, ldsa, b, ldb, sb, c, ldc, out_of(out_kind),
                         nullptr, 0, M, N, K, workspace, workspace_bytes, stream);
}

int fp8_block_gemm_e4m3_out(int a_kind, const void* a, int64_t lda, float* sa, int64_t ldsa,
                            const uint8_t* b, int64_t ldb, const float* sb, uint8_t* qc,
                            int64_t ldqc, float* sc, int64_t ldsc, int64_t M, int64_t N,
                            int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  return block_gemm_impl(a_kind, a, lda, sa, ldsa, b, ldb, sb, qc, ldqc, fp8bs::kOutE4M3, sc,
                         ldsc, M, N, K, workspace, workspace_bytes, stream);
}

int fp8_block_gemm_rowscaled(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                             const uint8_t* b, int64_t ldb, const float* sb, int64_t ldsb,
                             void* c, int64_t ldc, int out_kind, int64_t M, int64_t N, int64_t K,
                             void* stream) {
  if (out_kind != FP8BS_OUT_F32 && out_kind != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || K % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!a || !sa || !b || !sb || !c) return FP8BS_ERR_NULL;
  if (!operand_ld_ok(lda, K) || !operand_ld_ok(ldb, K) || ldc < N || ldsa < M || ldsb < N)
    return FP8BS_ERR_LAYOUT;
  const uintptr_t c_align = out_kind == FP8BS_OUT_F32 ? 4 : 2;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, c_align) || !aligned(sa, 4) ||
      !aligned(sb, 4))
    return FP8BS_ERR_LAYOUT;
  fp8bs::GemmArgs g{};
  g.a = a;
  g.lda = lda;
  g.sa = sa;
  g.ldsa = ldsa;
  g.b = b;
  g.ldb = ldb;
  g.sb = sb;
  g.sb_ld = ldsb;
  g.c = c;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  return hip_status(fp8bs::launch_block_gemm_rowscaled(g, out_of(out_kind),
                                                       static_cast<hipStream_t>(stream)));
}

int fp8_block_kgrouped_gemm_rowscaled(const uint8_t* a, int64_t lda, const float* sa,
                                      int64_t ldsa, const uint8_t* b, int64_t ldb,
                                      const float* sb, int64_t ldsb, void* c, int64_t ldc,
                                      int64_t c_group_stride, int out_kind,
                                      const int32_t* group_offsets, int64_t G, int64_t M,
                                      int64_t N, int64_t K_total, void* stream) {
  if (out_kind != FP8BS_OUT_F32 && out_kind != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
  if (G < 1 || G > kMaxGroups || M < 0 || N < 0 || K_total < 0 || K_total % kTile != 0)
    return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (!a || !sa || !b || !sb || !c || !group_offsets) return FP8BS_ERR_NULL;
  if (!operand_ld_ok(lda, K_total) || !operand_ld_ok(ldb, K_total) || ldc < N || ldsa < M ||
      ldsb < N || c_group_stride < (M - 1) * ldc + N)
    return FP8BS_ERR_LAYOUT;
  const uintptr_t c_align = out_kind == FP8BS_OUT_F32 ? 4 : 2;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, c_align) || !aligned(sa, 4) ||
      !aligned(sb, 4) || !aligned(group_offsets, 4))
    return FP8BS_ERR_LAYOUT;
  fp8bs::GemmArgs g{};
  g.a = a;
  g.lda = lda;
  g.sa = sa;
  g.ldsa = ldsa;
  g.b = b;
  g.ldb = ldb;
  g.sb = sb;
  g.sb_ld = ldsb;
  g.c = c;
  g.ldc = ldc;
  g.c_group_stride = c_group_stride;
  g.M = M;
  g.N = N;
  g.K = K_total;
  g.group_offsets = group_offsets;
  g.G = G;
  return hip_status(fp8bs::launch_kgrouped_gemm_rowscaled(g, out_of(out_kind),
                                                          static_cast<hipStream_t>(stream)));
}

int fp8_block_grouped_gemm(const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                           const uint8_t* b, int64_t ldb, int64_t b_group_stride,
                           const float* sb, void* c, int64_t ldc, int out_kind,
                           const int32_t* group_offsets, int64_t G, int64_t M_total, int64_t N,
                           int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (out_kind != FP8BS_OUT_F32 && out_kind != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
  return grouped_gemm_impl(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, c, ldc,
                           out_of(out_kind), nullptr, 0, group_offsets, G, M_total, N, K,
                           stream);
}

int fp8_block_grouped_gemm_e4m3_out(const uint8_t* a, int64_t lda, const float* sa,
                                    int64_t ldsa, const uint8_t* b, int64_t ldb,
                                    int64_t b_group_stride, const float* sb, uint8_t* qc,
                                    int64_t ldqc, float* sc, int64_t ldsc,
                                    const int32_t* group_offsets, int64_t G, int64_t M_total,
                                    int64_t N, int64_t K, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  return grouped_gemm_impl(a, lda, sa, ldsa, b, ldb, b_group_stride, sb, qc, ldqc,
                           fp8bs::kOutE4M3, sc, ldsc, group_offsets, G, M_total, N, K, stream);
}

int fp8_block_gemm_bf16_noalloc(const uint16_t* a, int64_t lda, float* sa, int64_t ldsa,
                                const uint8_t* b, int64_t ldb, const float* sb, void* c,
                                int64_t ldc, int out_kind, int64_t M, int64_t N, int64_t K,
                                void* stream) {
  if (out_kind != FP8BS_OUT_F32 && out_kind != FP8BS_OUT_BF16) return FP8BS_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || K % kTile != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) return FP8BS_OK;
  if (fp8bs_workspace_bytes(FP8BS_OP_GEMM_BF16, M, N, K, 0) > FP8BS_NOALLOC_SCRATCH_BYTES)
    return FP8BS_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e);
  return block_gemm_impl(FP8BS_A_BF16, a, lda, sa, ldsa, b, ldb, sb, c, ldc, out_of(out_kind),
                         nullptr, 0, M, N, K, ws, FP8BS_NOALLOC_SCRATCH_BYTES, stream);
}

size_t fp8bs_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t G) {
  (void)N;
  (void)G;
  if (M <= 0 || K <= 0) return 0;
  switch (op) {
    case FP8BS_OP_GEMM_BF16:
      return fused_q_bytes(M, K) + fused_s_bytes(M, K);
    default:
      return 0;
  }
}

const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL: return "a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "unsupported shape (negative size, K not a positive multiple of 128, or bad group count)";
    case FP8BS_ERR_LAYOUT: return "unsupported layout (leading dimension or pointer alignment)";
    case FP8BS_ERR_DTYPE: return "unknown a_kind, out_kind or mode";
    case FP8BS_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8BS_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int fp8bs_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
