// Launchers behind the C ABI (arguments already validated by abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace fp8bs {

// Launch kernel `k` and return the status of this launch alone.  (Reading
// hipGetLastError after a triple-chevron launch would also return, and
// clear, an error that an earlier unrelated call left pending, and report it
// as this call's failure.)  The arguments are converted to the kernel's
// parameter types first, so the argument array matches its signature.
template <class... P, class... A>
hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, hipStream_t stream,
                         A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count of the kernel");
  std::tuple<P...> vals(std::forward<A>(args)...);
  return std::apply(
      [&](auto&... v) {
        void* ptrs[] = {static_cast<void*>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, ptrs, 0, stream);
      },
      vals);
}

struct GemmArgs {
  const uint8_t* a;
  int64_t lda;
  const float* sa;
  int64_t ldsa;
  const uint8_t* b;
  int64_t ldb;
  int64_t b_group_stride;  // bytes between experts' weights (grouped only)
  const float* sb;
  int64_t sb_ld;  // block-scaled B: floats between consecutive 128-row bands of S_W (= K/128);
                  // row-scaled B: floats between consecutive K groups' rows of scales
  void* c;       // output: fp32, bf16 or E4M3 codes [M][ldc]
  int64_t ldc;
  float* sc;     // E4M3 output only: scale of row m, 128-column block nb at sc[nb*ldsc + m]
  int64_t ldsc;
  int64_t M;  // rows (dense) or M_total (grouped rows)
  int64_t N;
  int64_t K;  // contraction length (grouped along K: all groups' K_total)
  const int32_t* group_offsets;  // grouped only, device, G+1 entries
  int64_t G;
  int64_t c_group_stride;        // grouped along K: elements between the groups' outputs
};

hipError_t launch_quant_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds,
                            hipStream_t stream);

hipError_t launch_quant_act_delayed(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                    uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                    bool per_tensor, float* hist, int64_t ldh, int64_t H,
                                    int64_t step, uint32_t* stats, hipStream_t stream);

// M and N multiples of 128
hipError_t launch_quant_act_128x1_t(const uint16_t* x, int64_t M, int64_t N, int64_t ldx,
                                    uint8_t* qt, int64_t ldqt, float* st, int64_t ldst,
                                    hipStream_t stream);

// qt == nullptr: no transposed output
hipError_t launch_quant_w(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                          uint8_t* q, int64_t ldq, float* s, uint8_t* qt, int64_t ldqt,
                          float* st, hipStream_t stream);

// launch_quant_act and launch_quant_w (no transposed output) in one launch
hipError_t launch_quant_linear(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               const uint16_t* w, int64_t N, int64_t ldw, uint8_t* qw,
                               int64_t ldqw, float* sw, hipStream_t stream);

// Output element type of the GEMM kernels.
enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutE4M3 = 2 };

hipError_t launch_block_gemm(const GemmArgs& args, OutKind out, hipStream_t stream);

// B scaled per row and 128-K group: sb(n, kb) at sb[kb*sb_ld + n]
hipError_t launch_block_gemm_rowscaled(const GemmArgs& args, OutKind out, hipStream_t stream);

// Row-scaled B, grouped along K: group g contracts over K range
// [off[g], off[g+1]) (multiples of 128) into C + g*c_group_stride.
hipError_t launch_kgrouped_gemm_rowscaled(const GemmArgs& args, OutKind out,
                                          hipStream_t stream);

hipError_t launch_grouped_gemm(const GemmArgs& args, OutKind out, hipStream_t stream);

// Few-row GEMM (M <= kFewRows), fp32 or bf16 output.  fused (M <=
// kFewRowsFused): A is bf16 [M][lda], quantized per 1x128 tile inside the
// kernel (sa: optional scale output); otherwise A is E4M3 codes with input
// scales sa.
constexpr int64_t kFewRows = 64;
constexpr int64_t kFewRowsFused = 16;
hipError_t launch_few_rows_gemm(const void* a, int64_t lda, float* sa, int64_t ldsa, bool fused,
                                const uint8_t* b, int64_t ldb, const float* sb, void* c,
                                int64_t ldc, bool out_bf16, int64_t M, int64_t N, int64_t K,
                                hipStream_t stream);

}  // namespace fp8bs
