// Launchers of the block-scaled FP8 GEMM (kernel template in gemm_kernel.hpp).

#include "gemm_kernel.hpp"

namespace fp8bs {

namespace {
// BM, BN, waves along M, waves along N, LDS stages, tile-rows per L2 group
using DenseCfg = gemm::Cfg<256, 256, 2, 4, 2, 8>;
using GroupedCfg = gemm::Cfg<128, 128, 2, 2, 2, 8>;
}  // namespace

hipError_t launch_block_gemm(const GemmArgs& args, bool out_bf16, hipStream_t stream) {
  return gemm::launch<DenseCfg, false>(args, out_bf16, stream);
}

hipError_t launch_grouped_gemm(const GemmArgs& args, bool out_bf16, hipStream_t stream) {
  return gemm::launch<GroupedCfg, true>(args, out_bf16, stream);
}

}  // namespace fp8bs
