// Grouped expert GEMMs, bf16 weights and activations, fp32 accumulation on MFMA.
//
// Gate/up: h[row][n] = SiLU(sum_k x[tok(row)][k] Wg[n][k]) * (sum_k x[tok(row)][k] Wu[n][k]),
// with the token gather fused into the activation loads (GC-MoE, summary: grouped GEMM with fused
// SwiGLU).  Down: y[row][n] = sum_k h[row][k] Wd[n][k].  Shapes follow the live routing histogram
// ("Decoding the Skew ...", Abstract: sparse expert GEMMs whose shapes vary with routing).
//
// Two tile families, chosen per expert on the device (select.hip):
//  * stream: one workgroup = 4 wavefronts x 16 weight rows, all (<= 64) of an expert's rows.
//    Operand roles are swapped so the weight rows sit on the MFMA's 16-wide row side and the few
//    tokens on the column side (the same idea as GC-MoE's operand-swapped MMA); weights go straight
//    from HBM into MFMA registers, each element used once, 64 contiguous bytes per row per load.
//  * mfma: 128x128 output tiles, K-steps of 64 staged through double-buffered LDS with an XOR
//    swizzle (conflict-free ds_read_b128), 2x2 wavefronts of 64x64 (x2 for gate and up), MFMA
//    32x32x16.
// Both are persistent: a fixed grid pops tiles from a device queue (zeroed by the selection
// kernel), heaviest experts first, m-tiles of one weight tile adjacent in the queue.
#include "common.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ int find_seg(const Seg* __restrict__ segs, int nseg, int t) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].tile_base <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

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
// ------------------------------------------------------------------------------------------------
template <int MQ, bool GU>
__device__ __forceinline__ void stream_tile_bf16(const Seg& sg, int m0, int rows, int n0) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = sg.K, N = sg.N;
  const int nrow = n0 + wv * 16 + r16;  // this lane's weight row (A operand)
  const uint16_t* wg = static_cast<const uint16_t*>(sg.w0) + (size_t)nrow * K + kg * 8;
  const uint16_t* wu = GU ? static_cast<const uint16_t*>(sg.w1) + (size_t)nrow * K + kg * 8 : nullptr;
  const uint16_t* xr[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;  // padded columns re-read a valid row; never stored
    const int gr = sg.row0 + m0 + r;
    const int src = sg.tok ? sg.tok[gr] : gr;
    xr[q] = static_cast<const uint16_t*>(sg.a) + (size_t)src * K + kg * 8;
  }
  f32x4 acc0[MQ], acc1[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    acc0[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr int U = (MQ == 1) ? 8 : 4;
  const int nsteps = K / 32;
  int ks = 0;
  for (; ks + U <= nsteps; ks += U) {
    uint4 a0[U], a1[U], b[U][MQ];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a0[u] = *reinterpret_cast<const uint4*>(wg + (ks + u) * 32);
      if (GU) a1[u] = *reinterpret_cast<const uint4*>(wu + (ks + u) * 32);
#pragma unroll
      for (int q = 0; q < MQ; ++q) b[u][q] = *reinterpret_cast<const uint4*>(xr[q] + (ks + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        acc0[q] = mfma16(as_bf16x8(a0[u]), as_bf16x8(b[u][q]), acc0[q]);
        if (GU) acc1[q] = mfma16(as_bf16x8(a1[u]), as_bf16x8(b[u][q]), acc1[q]);
      }
  }
  for (; ks < nsteps; ++ks) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(wg + ks * 32);
    uint4 a1 = a0;
    if (GU) a1 = *reinterpret_cast<const uint4*>(wu + ks * 32);
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const uint4 b = *reinterpret_cast<const uint4*>(xr[q] + ks * 32);
      acc0[q] = mfma16(as_bf16x8(a0), as_bf16x8(b), acc0[q]);
      if (GU) acc1[q] = mfma16(as_bf16x8(a1), as_bf16x8(b), acc1[q]);
    }
  }
  // C[i][j]: i = weight row 4*kg + r (within this wave's 16), j = token r16 of group q
  uint16_t* out = static_cast<uint16_t*>(sg.out);
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
      *reinterpret_cast<uint2*>(out + (size_t)(sg.row0 + m0 + r) * N + n0 + wv * 16 + kg * 4) = pk;
    }
  }
}

template <bool GU>
__global__ __launch_bounds__(256) void gemm_stream_bf16(const Seg* __restrict__ segs,
                                                         int32_t* __restrict__ meta) {
  __shared__ int slot;
  const int nseg = meta[0], ntiles = meta[1];
  for (;;) {
    const int t = pop_tile(&meta[2], &slot);
    if (t >= ntiles) break;
    const Seg& sg = segs[find_seg(segs, nseg, t)];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * kStreamMaxRows;
    const int rows = min(kStreamMaxRows, sg.rows - m0);
    const int n0 = nt * kStreamBN;
    if (rows <= 16) stream_tile_bf16<1, GU>(sg, m0, rows, n0);
    else if (rows <= 32) stream_tile_bf16<2, GU>(sg, m0, rows, n0);
    else stream_tile_bf16<4, GU>(sg, m0, rows, n0);
  }
}

// ------------------------------------------------------------------------------------------------
// LDS-tiled MFMA family: BM x BN output tile, BK = 64, 4 wavefronts as 2 (rows) x 2 (columns)
// ------------------------------------------------------------------------------------------------
constexpr int BM = kMfmaBM, BN = kMfmaBN, BK = 64;

// byte offset of 16-byte chunk `ch` (0..7) of LDS row `r` (rows of BK bf16 = 128 B)
__device__ __forceinline__ int lds_off(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }

template <bool GU>
__device__ __forceinline__ void mfma_tile_bf16(const Seg& sg, int m0, int rows, int n0,
                                               uint8_t* lds) {
  constexpr int NW = GU ? 2 : 1;
  constexpr int ROWS = BM + NW * BN;      // LDS rows per stage: activations then weights
  constexpr int STAGE = ROWS * 128;       // bytes per stage
  constexpr int LPT = ROWS * 8 / 256;     // 16-byte loads per thread per stage
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int K = sg.K, N = sg.N;

  // per-thread global source rows for the tile loads
  const uint16_t* src[LPT];
  int ldsoff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, ch = c & 7;
    ldsoff[i] = lds_off(r, ch);
    if (r < BM) {
      int rr = r < rows ? r : rows - 1;
      const int gr = sg.row0 + m0 + rr;
      const int s = sg.tok ? sg.tok[gr] : gr;
      src[i] = static_cast<const uint16_t*>(sg.a) + (size_t)s * K + ch * 8;
    } else if (r < BM + BN) {
      src[i] = static_cast<const uint16_t*>(sg.w0) + (size_t)(n0 + r - BM) * K + ch * 8;
    } else {
      src[i] = static_cast<const uint16_t*>(sg.w1) + (size_t)(n0 + r - BM - BN) * K + ch * 8;
    }
  }

  f32x16 acc[NW][2][2];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[w][i][j][r] = 0.f;

  const int nk = K / BK;
  uint4 stg[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) stg[i] = *reinterpret_cast<const uint4*>(src[i]);
#pragma unroll
  for (int i = 0; i < LPT; ++i) *reinterpret_cast<uint4*>(lds + ldsoff[i]) = stg[i];
  __syncthreads();

  const int l32 = lane & 31, khalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) {
#pragma unroll
      for (int i = 0; i < LPT; ++i)
        stg[i] = *reinterpret_cast<const uint4*>(src[i] + (size_t)(kt + 1) * BK);
    }
    const uint8_t* st = lds + (kt & 1) * STAGE;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + khalf;
      bf16x8 bt[2], aw[NW][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wm * 64 + j * 32 + l32;
        bt[j] = as_bf16x8(*reinterpret_cast<const uint4*>(st + lds_off(r, ch)));
      }
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = BM + w * BN + wn * 64 + i * 32 + l32;
          aw[w][i] = as_bf16x8(*reinterpret_cast<const uint4*>(st + lds_off(r, ch)));
        }
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[w][i][j] = mfma32(aw[w][i], bt[j], acc[w][i][j]);
    }
    if (more) {
      uint8_t* dst = lds + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int i = 0; i < LPT; ++i) *reinterpret_cast<uint4*>(dst + ldsoff[i]) = stg[i];
    }
    __syncthreads();
  }

  // epilogue: lane holds C[8*(r/4) + 4*khalf + r%4][l32] of each 32x32 block
  uint16_t* out = static_cast<uint16_t*>(sg.out);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wm * 64 + j * 32 + l32;
    if (r >= rows) continue;
    uint16_t* orow = out + (size_t)(sg.row0 + m0 + r) * N + n0 + wn * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float g = acc[0][i][j][q * 4 + s];
          v[s] = GU ? swiglu(g, acc[NW - 1][i][j][q * 4 + s]) : g;
        }
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(orow + i * 32 + q * 8 + khalf * 4) = pk;
      }
  }
}

template <bool GU>
__global__ __launch_bounds__(256, 1) void gemm_mfma_bf16(const Seg* __restrict__ segs,
                                                          int32_t* __restrict__ meta) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int slot;
  const int nseg = meta[0], ntiles = meta[1];
  for (;;) {
    const int t = pop_tile(&meta[2], &slot);
    if (t >= ntiles) break;
    const Seg& sg = segs[find_seg(segs, nseg, t)];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * BM;
    mfma_tile_bf16<GU>(sg, m0, min(BM, sg.rows - m0), nt * BN, lds);
  }
}

constexpr int mfma_lds_bytes(bool gu) { return 2 * (BM + (gu ? 2 : 1) * BN) * 128; }

hipError_t launch_gemms_bf16(const SelectOut& o, int num_cus, hipStream_t s) {
  static bool attr_done = false;
  if (!attr_done) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mfma_bf16<true>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, mfma_lds_bytes(true));
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mfma_bf16<false>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, mfma_lds_bytes(false));
    attr_done = true;
  }
  for (int g = 0; g < 2; ++g) {
    const Seg* ss = o.segs + (size_t)(g * kNumFam + kFamStream) * kSegCap;
    int32_t* ms = o.meta + (g * kNumFam + kFamStream) * kMetaStride;
    const Seg* sm = o.segs + (size_t)(g * kNumFam + kFamMfma) * kSegCap;
    int32_t* mm = o.meta + (g * kNumFam + kFamMfma) * kMetaStride;
    if (g == kGemmGateUp) {
      gemm_stream_bf16<true><<<num_cus * 4, 256, 0, s>>>(ss, ms);
      gemm_mfma_bf16<true><<<num_cus, 256, mfma_lds_bytes(true), s>>>(sm, mm);
    } else {
      gemm_stream_bf16<false><<<num_cus * 4, 256, 0, s>>>(ss, ms);
      gemm_mfma_bf16<false><<<num_cus * 2, 256, mfma_lds_bytes(false), s>>>(sm, mm);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
