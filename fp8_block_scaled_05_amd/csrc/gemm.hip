// Launchers of the block-scaled FP8 GEMM (kernel template in gemm_kernel.hpp).
//
// Tile shapes by problem shape (measured on MI355X with the dense, grouped and
// few-row workloads):
// - large M: 256x256 tiles, 8 waves of 128x64, two LDS stages (128 KB); the
//   large tile halves the L2->LDS traffic per flop compared with 128x256,
//   which matters more than the deeper pipeline a smaller tile would allow;
//   the same shape serves the grouped path.  When the dense raster would end
//   in a partial round of workgroups, its last tiles run as pairs of
//   128x256 tiles (a half-length last round); a group whose last tile-row
//   holds at most 128 rows runs that row as 128x256 tiles;
// - few rows (decode-like, weight-bandwidth bound): short tiles so that the
//   weight matrix is spread over many workgroups and every weight byte is
//   read once; 1 wave along M; four LDS stages (three K groups in flight).
//   E4M3 output (quantized per 128 output columns) needs tiles of whole
//   128-column groups, so it takes the 64x128 tile for every M <= 64.
// - M > 64 with too few 256x256 tiles to fill the compute units: 128x256 or
//   64x128 tiles when they finish in fewer rounds of workgroups by the
//   estimate below (bitwise the same results: every tile shape sums each
//   output's K groups in the same order).
// The weight-gradient GEMM (B scaled per row and K group) uses the same tiles.

#include "gemm_kernel.hpp"

namespace fp8bs {

namespace {
// BM, BN, waves along M, waves along N, LDS stages, tile-rows per L2 group
using LargeCfg = gemm::Cfg<256, 256, 2, 4, 2, 4>;
// half-height tiles: a last partial round of the dense raster, and groups'
// last tile-rows of at most 128 rows
using LargeTail = gemm::Cfg<128, 256, 2, 4, 2, 4>;
using Rows32Cfg = gemm::Cfg<32, 32, 1, 2, 4, 1>;
using Rows64Cfg = gemm::Cfg<64, 128, 1, 4, 4, 1>;

// Tile shape for M > 64: the least estimated time, counted in rounds of
// workgroups (one workgroup per compute unit), a round of 256x256, 128x256
// and 64x128 (four-stage) tiles taking 100, 77 and 40 (relative times per
// round at equal K, measured on MI355X with one or two rounds); the 256x256
// launch runs a last partial round of at most half the compute units as
// 128x256 tiles, half a round.
enum class Tiles { kLarge, kHalf, kSmall };
Tiles pick_tiles(const GemmArgs& a) {
  const int64_t cus = gemm::device_cus();
  if (cus <= 0) return Tiles::kLarge;
  const int64_t tl = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const int64_t th = ((a.M + 127) / 128) * ((a.N + 255) / 256);
  const int64_t ts = ((a.M + 63) / 64) * ((a.N + 127) / 128);
  const int64_t tail = tl % cus;
  const int64_t cost_l =
      100 * (tl / cus) + (tail == 0 ? 0 : (tl > cus && 2 * tail <= cus) ? 50 : 100);
  const int64_t cost_h = 77 * ((th + cus - 1) / cus);
  const int64_t cost_s = 40 * ((ts + cus - 1) / cus);
  if (cost_l <= cost_h && cost_l <= cost_s) return Tiles::kLarge;
  return cost_h <= cost_s ? Tiles::kHalf : Tiles::kSmall;
}
}  // namespace

hipError_t launch_block_gemm(const GemmArgs& args, OutKind out, hipStream_t stream) {
  // E4M3 output quantizes whole 128-column tiles inside a workgroup: the
  // 32-column few-row tile cannot, so E4M3 output uses the 64x128 tile
  if (args.M <= 32 && out != kOutE4M3) return gemm::launch<Rows32Cfg, gemm::kDense>(args, out, stream);
  if (args.M <= 64) return gemm::launch<Rows64Cfg, gemm::kDense>(args, out, stream);
  switch (pick_tiles(args)) {
    case Tiles::kSmall: return gemm::launch<Rows64Cfg, gemm::kDense>(args, out, stream);
    case Tiles::kHalf: return gemm::launch<LargeTail, gemm::kDense>(args, out, stream);
    default: return gemm::launch<LargeCfg, gemm::kDense, LargeTail>(args, out, stream);
  }
}

hipError_t launch_block_gemm_rowscaled(const GemmArgs& args, OutKind out, hipStream_t stream) {
  using gemm::RowScaledB;
  if (args.M <= 32) return gemm::launch<RowScaledB<Rows32Cfg>, gemm::kDense>(args, out, stream);
  if (args.M <= 64) return gemm::launch<RowScaledB<Rows64Cfg>, gemm::kDense>(args, out, stream);
  switch (pick_tiles(args)) {
    case Tiles::kSmall:
      return gemm::launch<RowScaledB<Rows64Cfg>, gemm::kDense>(args, out, stream);
    case Tiles::kHalf:
      return gemm::launch<RowScaledB<LargeTail>, gemm::kDense>(args, out, stream);
    default:
      return gemm::launch<RowScaledB<LargeCfg>, gemm::kDense, RowScaledB<LargeTail>>(args, out,
                                                                                     stream);
  }
}

hipError_t launch_kgrouped_gemm_rowscaled(const GemmArgs& args, OutKind out,
                                          hipStream_t stream) {
  using gemm::RowScaledB;
  return gemm::launch<RowScaledB<LargeCfg>, gemm::kGroupK, RowScaledB<LargeTail>>(args, out,
                                                                                   stream);
}

hipError_t launch_grouped_gemm(const GemmArgs& args, OutKind out, hipStream_t stream) {
  return gemm::launch<LargeCfg, gemm::kGroupRows, LargeTail>(args, out, stream);
}

}  // namespace fp8bs
