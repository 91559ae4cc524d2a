// Device-side tile-configuration selection from the live routing histogram.
//
// "Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch" (Abstract):
// the best fused-MoE kernel changes with routing skew and token count, and static token-count
// buckets ignore the per-expert distribution that decides tile padding and memory reuse; the
// dispatch runtime reads the live histogram on the GPU, with no CPU-GPU synchronisation.
//
// Here the choice is made per expert, from its row count c_e, inside one workgroup that runs
// between the permutation and the GEMMs:
//   c_e <= 64  -> weight-streaming tiles: the expert's rows ride along while its weights stream
//                 from HBM once (decode-sized experts are bandwidth-bound: c_e FLOP per weight byte);
//   c_e  > 64  -> LDS-tiled MFMA tiles of 256 rows (padding only the last tile of the expert).
// Block-scaled fp8 experts always take the streaming family (up to 128 rows per pass).
// Experts with several m-tiles come first in their family's list, so the persistent GEMM queues
// start with the longest work.  Experts with no rows get no segment and their weights are never
// read.
#include "select_dev.h"

namespace moe {

__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a, SelectOut o) {
  select_block(a, o);
}

hipError_t launch_select(const SelectArgs& a, const SelectOut& o, hipStream_t s) {
  select_kernel<<<1, kSelMax, 0, s>>>(a, o);
  return hipGetLastError();
}

}  // namespace moe
