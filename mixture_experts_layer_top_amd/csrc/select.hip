// Device-side tile-configuration selection from the live routing histogram.
//
// "Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch" (Abstract):
// the best fused-MoE kernel changes with routing skew and token count, and static token-count
// buckets ignore the per-expert distribution that decides tile padding and memory reuse; the
// dispatch runtime reads the live histogram on the GPU, with no CPU-GPU synchronisation.
//
// Here the choice is made per expert and per GEMM, from the expert's row count c_e, inside one
// workgroup that runs between the permutation and the GEMMs:
//   down GEMM with c_e <= 8 -> weight-streaming tiles: the expert's rows ride along while its
//                 weights stream from HBM once (a handful of rows: c_e FLOP per weight byte) --
//                 unless the down GEMM's heavier experts fill a round of MFMA tiles by
//                 themselves: then the light ones join them on MFMA tiles;
//   otherwise -> LDS-tiled MFMA tiles of 256 weight rows by 64, 128 or 256 token rows (the tile
//                 height follows the rows the tile holds), so a light expert streams its weights
//                 through LDS once and pays MFMA time for at most 63 padding rows.
// Measured on 256-expert decode shapes: with short MFMA tiles, even one-row gate/up experts run
// faster on the MFMA family than on the streaming tiles as long as there are enough tiles, while
// the down GEMM (short K = d_ff) still prefers streaming for up to about 8 rows.
// An MFMA tile costs a whole K loop on one CU however few rows it holds: when a GEMM's MFMA tiles
// would fill fewer than 1.6 rounds of CUs and none of its experts holds more than 16 rows, the
// whole GEMM takes the streaming tiles, which spread each expert's weights over many workgroups
// (with one heavier expert it stays on MFMA: no GEMM is split between a streaming launch and an
// under-filled MFMA launch by this rule).  Block-scaled fp8 experts always take the
// streaming family (up to 32 rows per pass).  Inside an MFMA list, segments of full-height tiles come
// first and those of shorter tiles last (an expert's short last m-tile is a segment of its own), so
// the persistent kernel hands out the longest tiles first and the short ones fill the last round;
// when that round would leave CUs idle, its tiles are split in K (kernels.h).  Experts with no rows
// get no segment and their weights are never read.
#include "select_dev.h"

namespace moe {

__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a, SelectOut o) {
  select_block(a, o);
}

hipError_t launch_select(const SelectArgs& a, const SelectOut& o, hipStream_t s) {
  select_kernel<<<1, kSelThreads, 0, s>>>(a, o);
  return hipGetLastError();
}

}  // namespace moe
