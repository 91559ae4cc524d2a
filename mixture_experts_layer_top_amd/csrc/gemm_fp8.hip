// Grouped expert GEMMs with block-scaled fp8 (OCP e4m3) weights and activations.
//
// GC-MoE (summary) runs FP8 grouped GEMMs with block scales, fused SwiGLU, requantisation and
// optional shared experts for decode, where each rank holds 1-256 tokens and weight traffic
// dominates.  Here, per expert and per 128-wide K block kb:
//   P = sum_{k in kb} q_w[n][k] * q_x[row][k]      (exact in the fp32 MFMA accumulator)
//   acc[row][n] += P * (s_w[n/128][kb] * s_x[row][kb])
// with s_w the weight's 128x128 block scale and s_x the row's 1x128 activation scale.
//
// One workgroup = 4 wavefronts; weight rows on the MFMA's 16-wide row side, up to 32 token rows
// per pass on the column side (operand-swapped as in the bf16 streaming family); weights stream
// straight from HBM into MFMA registers (32 contiguous bytes per lane per 128-wide block), the
// next block's loads in flight while the current one is computed.
//   gate/up: 128 weight rows per workgroup (2 row groups of 16 per wavefront, gate and up), so the
//            workgroup owns one whole 128-column block of h: h = SiLU(g) * u is requantised per row
//            over that block (s = amax / 448, q = e4m3(h / s)) for the fp8 down GEMM.
//   down   : 64 weight rows per workgroup (16 per wavefront), bf16 output.
// MFMA: v_mfma_scale_f32_16x16x128_f8f6f4 with both formats e4m3 and unit E8M0 scales; the fp32
// block scales are applied to each 128-wide partial product.
#include "common.h"
#include "fp8_codec.h"
#include "kernels.h"

namespace moe {

constexpr int kFp8Rows = kStreamMaxRows8;  // token rows per pass (2 groups of 16)

__device__ __forceinline__ i32x8 as_i32x8(const uint4& lo, const uint4& hi) {
  i32x8 r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}


// Runs compute over the nkb K blocks.  Pipelined: the loads of block kb + 1 are issued before block
// kb is computed (two register buffers, unrolled by two so no buffer is copied); otherwise each
// block's loads are waited for before its MFMAs.
// (Pinning this loop's load groups with scheduling barriers and branch-free loads, which made the
// MXFP4 tiles 15-25% faster, measured neutral to 4% slower here: with two or more wavefronts per
// SIMD the other wavefronts cover the drained waits.)
template <bool PIPE, class Blk, class Load, class Compute>
__device__ __forceinline__ void k_blocks_pipelined(int nkb, Load& load, Compute& compute) {
  if (PIPE) {
    Blk b0, b1;
    load(b0, 0);
    int kb = 0;
    for (; kb + 1 < nkb; kb += 2) {
      load(b1, kb + 1);
      compute(b0);
      if (kb + 2 < nkb) load(b0, kb + 2);
      compute(b1);
    }
    if (kb < nkb) compute(b0);  // odd nkb: the last block sits in b0
  } else {
    for (int kb = 0; kb < nkb; ++kb) {
      Blk b;
      load(b, kb);
      compute(b);
    }
  }
}

// Gate/up tile: rows [m0, m0+rows) of segment sg (rows <= 16*MQ), weight rows n0 .. n0+127.
template <int MQ>
__device__ __forceinline__ void fp8_gateup_tile(const Seg& sg, int m0, int rows, int n0,
                                                float (*red)[kFp8Rows]) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = sg.K, N = sg.N, nkb = K / 128;
  // this lane's weight rows for row groups 0, 1
  uint32_t woff[2];
#pragma unroll
  // tiled weights (moe_fp8_tile): per 16-row block and 128-byte chunk of K, 2 KB ordered
  // [half][lane group][row][16 bytes], so lane kg * 16 + r16 reads its row's 32 bytes of the chunk
  // as two 16-byte loads 1 KB apart, and each load instruction reads 1 KB contiguously
  for (int g = 0; g < 2; ++g) woff[g] = (uint32_t)(n0 + wv * 32 + g * 16) * K + lane * 16;
  uint32_t xoff[MQ];
  int srow[MQ];  // activation row of token column r16 in group q (for its scale)
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;
    const int gr = sg.row0 + m0 + r;
    srow[q] = sg.tok ? gload_i32(sg.tok, gr) : gr;
    xoff[q] = (uint32_t)srow[q] * K + kg * 32;
  }
  const int nb = n0 / 128;  // weight scale block row (uniform)
  f32x4 ag[2][MQ], au[2][MQ];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      ag[g][q] = f32x4{0.f, 0.f, 0.f, 0.f};
      au[g][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // one 128-wide K block: weights, activations and their scales
  struct Blk { i32x8 wg[2], wu[2], xb[MQ]; float swg, swu, sx[MQ]; };
  auto load = [&](Blk& b, int kb) {
    const uint32_t ko = (uint32_t)kb * 128;
#pragma unroll
    for (int g = 0; g < 2; ++g) {  // (weights: non-temporal, see gload16_nt; -6% per layer)
      b.wg[g] = as_i32x8(gload16_nt(sg.w0, woff[g] + ko * 16), gload16_nt(sg.w0, woff[g] + ko * 16 + 1024));
      b.wu[g] = as_i32x8(gload16_nt(sg.w1, woff[g] + ko * 16), gload16_nt(sg.w1, woff[g] + ko * 16 + 1024));
    }
#pragma unroll
    for (int q = 0; q < MQ; ++q) b.xb[q] = as_i32x8(gload16(sg.a, xoff[q] + ko), gload16(sg.a, xoff[q] + ko + 16));
    b.swg = gload_f32(sg.s0, nb * nkb + kb);
    b.swu = gload_f32(sg.s1, nb * nkb + kb);
#pragma unroll
    for (int q = 0; q < MQ; ++q) b.sx[q] = gload_f32(sg.as, srow[q] * nkb + kb);
  };
  auto compute = [&](const Blk& b) {
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const float cg = b.swg * b.sx[q], cu = b.swu * b.sx[q];
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const f32x4 pg = mfma16_fp8(b.wg[g], b.xb[q], zero);
        const f32x4 pu = mfma16_fp8(b.wu[g], b.xb[q], zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ag[g][q][i] = fmaf(pg[i], cg, ag[g][q][i]);
          au[g][q][i] = fmaf(pu[i], cu, au[g][q][i]);
        }
      }
    }
  };
  k_blocks_pipelined<true, Blk>(nkb, load, compute);
  // SwiGLU, then per-row requantisation over this workgroup's 128 columns.
  // lane holds C[i = 4*kg + r][j = r16]: weight row n0 + wv*32 + g*16 + 4*kg + r, token column j.
  float h[2][MQ][4];
  float amax[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    amax[q] = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[g][q][i] = swiglu(ag[g][q][i], au[g][q][i]);
        amax[q] = fmaxf(amax[q], fabsf(h[g][q][i]));
      }
    amax[q] = fmaxf(amax[q], __shfl_xor(amax[q], 16));
    amax[q] = fmaxf(amax[q], __shfl_xor(amax[q], 32));
  }
  __syncthreads();  // red[] may still be read by the previous tile
#pragma unroll
  for (int q = 0; q < MQ; ++q)
    if (kg == 0) red[wv][q * 16 + r16] = amax[q];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    const int r = q * 16 + r16;
    float m = fmaxf(fmaxf(red[0][q * 16 + r16], red[1][q * 16 + r16]),
                    fmaxf(red[2][q * 16 + r16], red[3][q * 16 + r16]));
    float s = m / 448.0f;
    if (m == 0.0f || s == 0.0f) s = 1.0f;
    const float inv = 1.0f / s;
    if (r < rows) {
      const size_t orow = (size_t)(sg.row0 + m0 + r);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t pk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk |= uint32_t(e4m3_encode(h[g][q][i] * inv)) << (8 * i);
        gstore4(sg.out, orow * N + n0 + wv * 32 + g * 16 + kg * 4, pk);
      }
      if (wv == 0 && kg == 0) gstore_f32(sg.outs, orow * (N / 128) + n0 / 128, s);
    }
  }
}

// Down tile: rows [m0, m0+rows) (rows <= 16*MQ), weight rows n0 .. n0+63, bf16 output.
template <int MQ>
__device__ __forceinline__ void fp8_down_tile(const Seg& sg, int m0, int rows, int n0) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = sg.K, N = sg.N, nkb = K / 128;
  const uint32_t woff = (uint32_t)(n0 + wv * 16) * K + lane * 16;  // tiled weights, as gate/up
  uint32_t xoff[MQ];
  int srow[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;
    srow[q] = sg.row0 + m0 + r;
    xoff[q] = (uint32_t)srow[q] * K + kg * 32;
  }
  const int nb = (n0 + wv * 16) / 128;
  f32x4 acc[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  struct Blk { i32x8 w, xb[MQ]; float sw, sx[MQ]; };
  auto load = [&](Blk& b, int kb) {
    const uint32_t ko = (uint32_t)kb * 128;
    b.w = as_i32x8(gload16_nt(sg.w0, woff + ko * 16), gload16_nt(sg.w0, woff + ko * 16 + 1024));
#pragma unroll
    for (int q = 0; q < MQ; ++q) b.xb[q] = as_i32x8(gload16(sg.a, xoff[q] + ko), gload16(sg.a, xoff[q] + ko + 16));
    b.sw = gload_f32(sg.s0, nb * nkb + kb);
#pragma unroll
    for (int q = 0; q < MQ; ++q) b.sx[q] = gload_f32(sg.as, srow[q] * nkb + kb);
  };
  auto compute = [&](const Blk& b) {
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const float c = b.sw * b.sx[q];
      const f32x4 p = mfma16_fp8(b.w, b.xb[q], zero);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[q][i] = fmaf(p[i], c, acc[q][i]);
    }
  };
  k_blocks_pipelined<true, Blk>(nkb, load, compute);
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    const int r = q * 16 + r16;
    if (r < rows) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[q][0], acc[q][1]);
      pk.y = pack_bf16x2(acc[q][2], acc[q][3]);
      gstore8(sg.out, ((size_t)(sg.row0 + m0 + r) * N + n0 + wv * 16 + kg * 4) * 2, pk);
    }
  }
}

// Persistent, as the bf16 streaming kernel: workgroup b takes tile b first, then pops tiles
// gridDim.x, gridDim.x + 1, ... from the list's queue counter; segment bases are staged in LDS.
template <bool GU>
__global__ __launch_bounds__(256) void gemm_stream_fp8(const Seg* __restrict__ segs,
                                                        int32_t* __restrict__ meta) {
  __shared__ int slot;
  __shared__ int seg_base[kSegCap];
  __shared__ float red[4][kFp8Rows];
  const int nseg = meta[0], ntiles = meta[1];
  if ((int)blockIdx.x >= ntiles) return;
  for (int i = threadIdx.x; i < nseg; i += 256) seg_base[i] = segs[i].tile_base;
  __syncthreads();
  int t = blockIdx.x;
  for (;;) {
    const Seg& sg = segs[__builtin_amdgcn_readfirstlane(find_seg_lds(seg_base, nseg, t))];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * kFp8Rows;
    const int rows = min(kFp8Rows, sg.rows - m0);
    static_assert(kFp8Rows == 32, "token groups per pass");
    if (GU) {
      const int n0 = nt * kStream8BNGateUp;
      if (rows <= 16) fp8_gateup_tile<1>(sg, m0, rows, n0, red);
      else fp8_gateup_tile<2>(sg, m0, rows, n0, red);
    } else {
      const int n0 = nt * kStream8BNDown;
      if (rows <= 16) fp8_down_tile<1>(sg, m0, rows, n0);
      else fp8_down_tile<2>(sg, m0, rows, n0);
    }
    if (threadIdx.x == 0) slot = atomicAdd(&meta[kMetaQueue], 1);
    __syncthreads();
    t = gridDim.x + __builtin_amdgcn_readfirstlane(slot);
    __syncthreads();
    if (t >= ntiles) break;
  }
}

hipError_t launch_gemms_fp8(const SelectOut& o, int g, int num_cus, int64_t max_rows, bool stream,
                            bool mfma, hipStream_t s) {
  const Seg* ss = o.segs + (size_t)(g * kNumFam + kFamStream) * kSegCap;
  int32_t* ms = o.meta + (g * kNumFam + kFamStream) * kMetaStride;
  if (stream) {
    // persistent grid: six workgroups per CU while every expert fits one 32-row pass (fp8
    // DeepSeek-V3-shaped layer at T = 32: 1.05 -> 1.03 ms), else four (at T = 128 six were 1%
    // slower)
    const int grid = (max_rows <= kStreamMaxRows8 ? 6 : 4) * num_cus;
    if (g == kGemmGateUp) gemm_stream_fp8<true><<<grid, 256, 0, s>>>(ss, ms);
    else gemm_stream_fp8<false><<<grid, 256, 0, s>>>(ss, ms);
  }
  if (mfma)
    launch_mfma_fp8(o.segs + (size_t)(g * kNumFam + kFamMfma) * kSegCap,
                    o.meta + (g * kNumFam + kFamMfma) * kMetaStride, g, num_cus, s);
  return hipGetLastError();
}

}  // namespace moe
