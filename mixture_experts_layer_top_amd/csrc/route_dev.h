// Top-k routing of one token by one wavefront (shared by the routing kernel and the fused decode
// front end).  Lane l holds logits l, l+64, ...; each of the k rounds takes every lane's best
// untaken candidate and reduces over the wavefront with a butterfly on the total order
// (value desc, id asc); IEEE comparisons make -0.0 and +0.0 a tie.  Weights: expf of the gap to
// the largest selected logit, divided by their sum (softmax renormalised over the selected k).
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ bool route_better(float a, int ia, float b, int ib) {
  return a > b || (a == b && ia < ib);
}

// Routes token t; lane 0 writes ids/w (and the ids to lds_ids[t*k + j] if lds_ids is not null).
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int* lds_ids) {
  const int lane = threadIdx.x & 63;
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
        if (cand && (bi == 0x7fffffff || route_better(v[i], e, best, bi))) {
          best = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bi, off);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || route_better(ob, oi, best, bi))) {
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
        if (lds_ids) lds_ids[t * k + j] = sel_i[j];
      }
    }
  }
}

// Block-wide exclusive scan of NA values per thread (blockDim.x = 64 * NWAVE), with totals.
// `lds` holds NWAVE * NA ints.  Contains __syncthreads: every thread of the block must call it.
template <int NA, int NWAVE>
__device__ __forceinline__ void block_scan(const int (&v)[NA], int (&excl)[NA], int (&tot)[NA],
                                           int* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) incl[i] = v[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int u = __shfl_up(incl[i], off);
      if (lane >= off) incl[i] += u;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds[wv * NA + i] = incl[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    int base = 0, all = 0;
    for (int w = 0; w < NWAVE; ++w) {
      const int s = lds[w * NA + i];
      base += (w < wv) ? s : 0;
      all += s;
    }
    excl[i] = base + incl[i] - v[i];
    tot[i] = all;
  }
  __syncthreads();
}

}  // namespace moe
