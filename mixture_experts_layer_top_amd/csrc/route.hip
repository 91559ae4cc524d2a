// Top-k routing with renormalised softmax gate weights.
//
// Routing result: per token, the k experts with the largest router logits, ties to the lower expert
// id (Weave, Abstract: the layer's volumes follow from the routing result; the pages leave the
// score function open -- this is the softmax renormalised over the selected k).
//
// One wavefront per token.  Lane l holds logits l, l+64, ... (coalesced row load).  Each of the k
// rounds takes every lane's best untaken candidate and reduces over the wavefront with a butterfly
// on the total order (value desc, id asc); IEEE comparisons make -0.0 and +0.0 a tie.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ bool better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? row[e] : 0.0f;
  }
  uint32_t taken = 0;
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      float best = 0.0f;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const int e = lane + 64 * i;
        const bool cand = e < E && !((taken >> i) & 1u);
        if (cand && (bi == 0x7fffffff || better(v[i], e, best, bi))) {
          best = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || better(ob, oi, best, bi))) {
          best = ob;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      sel_v[j] = best;
      sel_i[j] = bi;
    }
  }
  if (lane == 0) {
    float ex[8];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ex[j] = expf(sel_v[j] - sel_v[0]);
        sum += ex[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ids[(size_t)t * k + j] = sel_i[j];
        w[(size_t)t * k + j] = ex[j] / sum;
      }
    }
  }
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
