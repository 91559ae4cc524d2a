// Top-k routing of one token by one wavefront (shared by the routing kernel and the fused decode
// front end).  Lane l holds logits l, l+64, ...; each of the k rounds selects the best untaken
// candidate in the total order (value desc, id asc; -0.0 and +0.0 tie).  Weights: expf of the gap
// to the largest selected logit, divided by their sum (softmax renormalised over the selected k).
#pragma once

#include "common.h"

namespace moe {

// Candidate keys: the logit's bits mapped so that unsigned order is IEEE order (+0.0 and -0.0 are
// first made the same value, so they tie).  Every finite logit maps above 0, and key 0 marks "no
// candidate" (past E, or already selected).
__device__ __forceinline__ uint32_t route_ordered(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);  // -0.0 + 0.0 = +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float route_unordered(uint32_t h) {
  return __uint_as_float((h & 0x80000000u) ? (h & 0x7fffffffu) : ~h);
}

// Largest key of the wavefront: DPP max inside rows of 16 lanes (swap neighbours, swap pairs,
// mirror halves, mirror rows: every lane then holds its row's largest), then across the four rows
// through scalar registers.
__device__ __forceinline__ uint32_t route_wave_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xb1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4e, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xf, 0xf, false));  // row_half_mirror
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xf, 0xf, false));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(m, 0), r1 = __builtin_amdgcn_readlane(m, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(m, 32), r3 = __builtin_amdgcn_readlane(m, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Routes token t; lane 0 writes ids/w when they are not null, and the ids to lds_ids[t*k + j] when
// lds_ids is not null.  Each of the k rounds takes the largest remaining key of the wavefront, and
// among the candidates holding it (equal logits) the lowest expert id: lane l holds experts l,
// l + 64, ..., so that is the lowest set lane of the first of its VPL ballots that has one.
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int t, int E, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                            int* lds_ids) {
  const int lane = threadIdx.x & 63;
  const float* row = logits + (size_t)t * E;
  uint32_t kh[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    kh[i] = e < E ? route_ordered(row[e]) : 0u;
  }
  float sel_v[8];
  int sel_i[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < k) {
      uint32_t m = kh[0];
#pragma unroll
      for (int i = 1; i < VPL; ++i) m = max(m, kh[i]);
      const uint32_t best = route_wave_max(m);
      int bi = -1;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const uint64_t hit = __ballot(kh[i] == best);
        if (bi < 0 && hit != 0) bi = 64 * i + (__ffsll((unsigned long long)hit) - 1);
      }
      // the selected candidate drops out of later rounds
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (lane + 64 * i == bi) kh[i] = 0u;
      sel_v[j] = route_unordered(best);
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
        if (ids) ids[(size_t)t * k + j] = sel_i[j];
        if (w) w[(size_t)t * k + j] = ex[j] / sum;
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
