// Top-k routing with renormalised softmax gate weights.
//
// Routing result: per token, the k experts with the largest router logits, ties to the lower expert
// id (Weave, Abstract: the layer's volumes follow from the routing result; the pages leave the
// score function open -- this is the softmax renormalised over the selected k).
//
// One wavefront per token (route_dev.h).
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<VPL>(logits, t, E, k, ids, w, nullptr);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  else
    route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, w);
  return hipGetLastError();
}

}  // namespace moe
