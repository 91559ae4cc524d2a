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

// Inclusive prefix sum inside each row of 16 lanes (DPP row shifts; lanes shifted in from outside
// the row read 0).
__device__ __forceinline__ int row16_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wavefront: row scans, then lane 15 is broadcast
// into rows 1 and 3 and lane 31 into rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x = row16_incl_scan(x);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// LDS ints block_scan needs for NA values per thread.
constexpr int block_scan_lds(int na) { return 33 * na; }

// Block-wide exclusive scan of NA values per thread (blockDim.x = 64 * NWAVE, NWAVE <= 16), with
// totals.  Wavefront scans, then one 16-lane row scan per value over the wavefront totals.
// `lds` holds block_scan_lds(NA) ints.  Contains __syncthreads: every thread of the block must
// call it.
template <int NA, int NWAVE>
__device__ __forceinline__ void block_scan(const int (&v)[NA], int (&excl)[NA], int (&tot)[NA],
                                           int* lds) {
  static_assert(NWAVE <= 16 && NA * 16 <= 64 * NWAVE, "block_scan shape");
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) incl[i] = wave_incl_scan(v[i]);
  // lds[i * 16 + w]: wavefront totals (rows of waves that do not exist are 0)
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NA; ++i) lds[i * 16 + wv] = incl[i];
  }
  if (NWAVE < 16 && threadIdx.x < NA * 16 && (threadIdx.x & 15) >= NWAVE) lds[threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x < NA * 16) {  // thread i * 16 + w: value i, wavefront w
    const int s = lds[threadIdx.x];
    const int inc = row16_incl_scan(s);
    lds[NA * 16 + threadIdx.x] = inc - s;
    if ((threadIdx.x & 15) == 15) lds[2 * NA * 16 + (threadIdx.x >> 4)] = inc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    excl[i] = lds[NA * 16 + i * 16 + wv] + incl[i] - v[i];
    tot[i] = lds[2 * NA * 16 + i];
  }
  __syncthreads();
}

}  // namespace moe
