// Device-side tile-configuration selection from the live routing histogram.
//
// "Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch" (Abstract):
// the best fused-MoE kernel changes with routing skew and token count, and static token-count
// buckets ignore the per-expert distribution that decides tile padding and memory reuse; the
// dispatch runtime reads the live histogram on the GPU, with no CPU-GPU synchronisation.
//
// Here the choice is made per expert and per GEMM, from the expert's row count c_e, inside one
// workgroup that runs between the permutation and the GEMMs:
//   c_e <= 8 (gate/up) or 16 (down) -> weight-streaming tiles: the expert's rows ride along while
//                 its weights stream from HBM once (a handful of rows: c_e FLOP per weight byte);
//   above that -> LDS-tiled MFMA tiles of 256 rows.  A tile runs MFMAs only for its 32-row blocks
//                 that hold rows, so a light expert's tile streams its weights through LDS once and
//                 costs MFMA time in proportion to its rows.
// An MFMA tile costs a whole K loop on one CU however few rows it holds: when a GEMM's MFMA tiles
// would not fill two rounds of CUs, its experts of up to 64 rows stay on the streaming tiles.
// The streaming family re-reads an expert's rows from L2 for every 16 weight rows, which is what
// caps it at a few rows per expert.  For a down GEMM with long K (d_ff >= 4096) an expert whose
// last 256-row m-tile would hold at most 64 rows sends those rows to the streaming family: such a
// tile costs nearly a full tile's LDS-load time, and a few of them can add a whole round of tiles.  Block-scaled fp8 experts always take the streaming family (up
// to 128 rows per pass).  Inside a (GEMM, family) list, experts with several m-tiles come first
// ("heavy"); the MFMA kernels spread the light tiles evenly between the heavy ones, so HBM-bound
// and MFMA-bound tiles run side by side.  Experts with no rows get no segment and their weights are
// never read.
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
