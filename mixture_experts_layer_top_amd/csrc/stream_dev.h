// Pieces shared by the weight-streaming tile kernels (bf16, MXFP4 and MXFP4 x MXFP8 weights): the
// queue pop of the persistent loop and the split-K reduction with the bf16 epilogue.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Pops the next tile index for the whole workgroup.
__device__ __forceinline__ int pop_tile(int32_t* queue, int* slot) {
  if (threadIdx.x == 0) *slot = atomicAdd(queue, 1);
  __syncthreads();
  const int t = *slot;
  __syncthreads();
  return t;
}

// ------------------------------------------------------------------------------------------------
// weight-streaming family
//
// One workgroup = 16 weight rows split four ways in K, or 32 split two ways (gate/up: as many
// gate and up rows), and up to 64 rows of an expert's segment; the partial sums meet in LDS
// (added in a fixed order, so results are deterministic).  Small tiles give decode-sized layers
// enough workgroups (T = 1, 8 experts: 1024 gate/up tiles), and each wavefront reads only its share
// of the activations.  Loads are double-buffered in registers across unrolled batches of K-steps.
// ------------------------------------------------------------------------------------------------
// Split-K reduction and epilogue of a streaming tile: in each group of 16 weight rows, wavefronts
// kw = 1..WK-1 park their partials in LDS and wavefront kw = 0 adds them in order (slots
// grp * (WK - 1) + kw - 1, at most 3), then applies SwiGLU (gate/up) and stores bf16.  n0 is the
// first column of the calling wavefront's group of 16.
template <int MQ, bool GU, int WK, bool COH = false>
__device__ __forceinline__ void stream_tile_finish(const Seg& sg, int m0, int rows, int n0,
                                                   float* red, f32x4 (&acc0)[MQ], f32x4 (&acc1)[MQ]) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int grp = wv / WK, kw = wv % WK;
  const int N = sg.N;
  constexpr int NV = MQ * 4 * (GU ? 2 : 1);  // floats per lane
  if (WK > 1) __syncthreads();  // red[] may still be read by the previous tile
  if (WK > 1 && kw > 0) {
    float* dst = red + ((grp * (WK - 1) + kw - 1) * NV) * 64 + lane;
#pragma unroll
    for (int q = 0; q < MQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[(q * 4 + i) * 64] = acc0[q][i];
        if (GU) dst[(MQ * 4 + q * 4 + i) * 64] = acc1[q][i];
      }
  }
  if (WK > 1) {
    __syncthreads();
    if (kw != 0) return;
  }
#pragma unroll
  for (int w = 0; w < WK - 1; ++w) {
    const float* src = red + ((grp * (WK - 1) + w) * NV) * 64 + lane;
#pragma unroll
    for (int q = 0; q < MQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc0[q][i] += src[(q * 4 + i) * 64];
        if (GU) acc1[q][i] += src[(MQ * 4 + q * 4 + i) * 64];
      }
  }
  // C[i][j]: i = weight row 4*kg + r, j = token r16 of group q
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    const int r = q * 16 + r16;
    if (r < rows) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = GU ? swiglu(acc0[q][i], acc1[q][i]) : acc0[q][i];
      uint2 pk;
      pk.x = pack_bf16x2(v[0], v[1]);
      pk.y = pack_bf16x2(v[2], v[3]);
      const size_t off = ((size_t)(sg.row0 + m0 + r) * N + n0 + kg * 4) * 2;
      if (COH) gstore8_coh(sg.out, off, pk);  // (read by other XCDs in the same launch)
      else gstore8(sg.out, off, pk);
    }
  }
}

}  // namespace moe
