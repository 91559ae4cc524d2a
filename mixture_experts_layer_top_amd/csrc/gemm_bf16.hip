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
  const void* wg = sg.w0;
  const void* wu = GU ? sg.w1 : sg.w0;
  const void* xa = sg.a;
  const uint32_t woff = (uint32_t)nrow * K * 2 + kg * 16;
  uint32_t xoff[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;  // padded columns re-read a valid row; never stored
    const int gr = sg.row0 + m0 + r;
    const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
    xoff[q] = (uint32_t)src * K * 2 + kg * 16;
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
      const uint32_t ko = (uint32_t)(ks + u) * 64;
      a0[u] = gload16(wg, woff + ko);
      if (GU) a1[u] = gload16(wu, woff + ko);
#pragma unroll
      for (int q = 0; q < MQ; ++q) b[u][q] = gload16(xa, xoff[q] + ko);
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
    const uint32_t ko = (uint32_t)ks * 64;
    const uint4 a0 = gload16(wg, woff + ko);
    uint4 a1 = a0;
    if (GU) a1 = gload16(wu, woff + ko);
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const uint4 b = gload16(xa, xoff[q] + ko);
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
  if (ntiles == 0) return;
  for (;;) {
    const int t = __builtin_amdgcn_readfirstlane(pop_tile(&meta[kMetaQueue], &slot));
    if (t >= ntiles) break;
    const Seg& sg = segs[__builtin_amdgcn_readfirstlane(find_seg(segs, nseg, t))];
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
// LDS-tiled MFMA family
//
// Tile: 256 token rows x 256 weight rows (gate/up: 128 gate + 128 up rows -> 128 h columns; down:
// 256 y columns), K-steps of 64 through two LDS stages of 64 KB (rows of 128 B, 16-byte chunks
// XOR-swizzled by row so ds_read_b128 is conflict-free).  4 wavefronts as 2 (tokens) x 2 (weights),
// each 128 x 128 with MFMA 32x32x16: 16 accumulator blocks, 4 A and 4 B fragments per k-substep,
// every fragment reused 4 times.  Global -> LDS through registers, one K-step ahead; LDS -> register
// fragments one k-substep ahead.  Bases are wavefront-uniform (scalar), per-lane offsets 32-bit.
//
// Scheduling: one persistent workgroup per CU.  The tile order puts the m-tiles of one weight tile
// next to each other; consecutive runs of (CUs per XCD) tiles go to one XCD, so tiles that share
// weight and activation tiles run side by side on the same L2.  Each XCD has its own queue; a
// workgroup whose queue is empty takes work from the other XCDs' queues.
// ------------------------------------------------------------------------------------------------
constexpr int BM = kMfmaBM, BK = 64;
constexpr int BNW = 256;                 // weight rows per tile
constexpr int LROWS = BM + BNW;          // LDS rows per stage
constexpr int STAGE = LROWS * 128;       // bytes per stage (64 KB)
constexpr int LPT = LROWS * 8 / 256;     // 16-byte global loads per thread per stage (16)
constexpr int kMfmaLds = 2 * STAGE;

// byte offset of 16-byte chunk `ch` (0..7) of LDS row `r` (rows of BK bf16 = 128 B)
__device__ __forceinline__ int lds_off(int r, int ch) { return r * 128 + ((ch ^ (r & 7)) << 4); }


template <bool GU>
__device__ __forceinline__ void mfma_tile_bf16(const Seg& sg, int m0, int rows, int n0,
                                               uint8_t* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv & 1, wn = wv >> 1;
  const int K = sg.K, N = sg.N;
  const uint32_t rowbytes = (uint32_t)K * 2;
  const char* abase = static_cast<const char*>(sg.a);
  const char* w0 = static_cast<const char*>(sg.w0);
  const char* w1 = static_cast<const char*>(GU ? sg.w1 : sg.w0);

  // Load slot i of this thread: LDS row 32*i + tid/8, chunk tid%8.  Slots 0..7 are token rows,
  // 8..15 weight rows (gate/up: 8..11 gate, 12..15 up).
  const int rsub = tid >> 3, ch = tid & 7;
  const uint32_t lds0 = lds_off(rsub, ch);
  uint32_t off[LPT];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = 32 * i + rsub;
    r = r < rows ? r : rows - 1;  // padded rows re-read a valid row and are never stored
    const int gr = sg.row0 + m0 + r;
    const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
    off[i] = (uint32_t)src * rowbytes + ch * 16;
  }
#pragma unroll
  for (int i = 8; i < 16; ++i) {
    int wr;
    if (GU) wr = n0 + 32 * ((i - 8) & 3) + rsub;  // gate rows (i < 12) or up rows (i >= 12)
    else wr = n0 + 32 * (i - 8) + rsub;
    wr = wr < N ? wr : N - 1;  // half-full edge tile of the down GEMM
    off[i] = (uint32_t)wr * rowbytes + ch * 16;
  }

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  uint4 stg[LPT];
  auto gload = [&](int kt) {
    const uint32_t ko = (uint32_t)kt * (BK * 2);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const char* base = i < 8 ? abase : ((!GU || i < 12) ? w0 : w1);
      stg[i] = gload16(base, off[i] + ko);
    }
  };
  auto lstore = [&](int stage) {
    uint8_t* dst = lds + stage * STAGE + lds0;
#pragma unroll
    for (int i = 0; i < LPT; ++i) *reinterpret_cast<uint4*>(dst + i * 32 * 128) = stg[i];
  };

  const int l32 = lane & 31, khalf = lane >> 5;
  // LDS rows of this wave's fragments: A (weights) blocks a = 0..3, B (tokens) blocks b = 0..3
  int arow[4], brow[4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
    arow[a] = GU ? (BM + (a < 2 ? 0 : 128) + wn * 64 + (a & 1) * 32 + l32)
                 : (BM + wn * 128 + a * 32 + l32);
#pragma unroll
  for (int b = 0; b < 4; ++b) brow[b] = wm * 128 + b * 32 + l32;

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  if (nk > 1) gload(1);

  for (int kt = 0; kt < nk; ++kt) {
    const uint8_t* st = lds + (kt & 1) * STAGE;
    bf16x8 fa[2][4], fb[2][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
      fa[0][a] = as_bf16x8(*reinterpret_cast<const uint4*>(st + lds_off(arow[a], khalf)));
#pragma unroll
    for (int b = 0; b < 4; ++b)
      fb[0][b] = as_bf16x8(*reinterpret_cast<const uint4*>(st + lds_off(brow[b], khalf)));
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      if (kk + 1 < BK / 16) {
        const int c2 = (kk + 1) * 2 + khalf;
#pragma unroll
        for (int a = 0; a < 4; ++a)
          fa[nxt][a] = as_bf16x8(*reinterpret_cast<const uint4*>(st + lds_off(arow[a], c2)));
#pragma unroll
        for (int b = 0; b < 4; ++b)
          fb[nxt][b] = as_bf16x8(*reinterpret_cast<const uint4*>(st + lds_off(brow[b], c2)));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(fa[cur][a], fb[cur][b], acc[a][b]);
    }
    if (kt + 1 < nk) {
      lstore((kt + 1) & 1);
      if (kt + 2 < nk) gload(kt + 2);
    }
    __syncthreads();
  }

  // epilogue: lane holds C[8*(r/4) + 4*khalf + r%4][l32] of each 32x32 block (rows = weights)
  uint16_t* out = static_cast<uint16_t*>(sg.out);
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int r = wm * 128 + b * 32 + l32;
    if (r >= rows) continue;
    uint16_t* orow = out + (size_t)(sg.row0 + m0 + r) * N;
    if (GU) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c0 = n0 + wn * 64 + a * 32 + khalf * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = swiglu(acc[a][b][q * 4 + s], acc[a + 2][b][q * 4 + s]);
          uint2 pk;
          pk.x = pack_bf16x2(v[0], v[1]);
          pk.y = pack_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(orow + c0 + q * 8) = pk;
        }
      }
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int cb = n0 + wn * 128 + a * 32;
        if (cb >= N) continue;
        const int c0 = cb + khalf * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[a][b][q * 4 + 0], acc[a][b][q * 4 + 1]);
          pk.y = pack_bf16x2(acc[a][b][q * 4 + 2], acc[a][b][q * 4 + 3]);
          *reinterpret_cast<uint2*>(orow + c0 + q * 8) = pk;
        }
      }
    }
  }
}

// Next tile for this workgroup from the per-XCD queues (see the scheduling note above), or -1.
// `q` is the workgroup's current queue offset (0 = its own XCD), kept across calls.
__device__ __forceinline__ int pop_tile_xcd(int32_t* queues, int ntiles, int chunk, int* slot,
                                            int& q) {
  const int xcd = blockIdx.x % kXcds;
  while (q < kXcds) {
    const int x = (xcd + q) % kXcds;
    if (threadIdx.x == 0) {
      const int i = atomicAdd(&queues[x], 1);
      *slot = (i / chunk) * (chunk * kXcds) + x * chunk + (i % chunk);
    }
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(*slot);
    __syncthreads();
    if (t < ntiles) return t;
    ++q;
  }
  return -1;
}

template <bool GU>
__global__ __launch_bounds__(256, 1) void gemm_mfma_bf16(const Seg* __restrict__ segs,
                                                          int32_t* __restrict__ meta) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int slot;
  const int nseg = meta[0], ntiles = meta[1];
  if (ntiles == 0) return;
  const int chunk = max(1, (int)gridDim.x / kXcds);
  int q = 0;
  for (;;) {
    const int t = pop_tile_xcd(meta + kMetaQueue, ntiles, chunk, &slot, q);
    if (t < 0) break;
    const int si = __builtin_amdgcn_readfirstlane(find_seg(segs, nseg, t));
    const Seg& sg = segs[si];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * BM;
    mfma_tile_bf16<GU>(sg, m0, min(BM, sg.rows - m0), nt * (GU ? kMfmaBNGateUp : kMfmaBNDown), lds);
  }
}

hipError_t launch_gemms_bf16(const SelectOut& o, int g, int num_cus, hipStream_t s) {
  static bool attr_done = false;
  if (!attr_done) {
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mfma_bf16<true>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaLds);
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_mfma_bf16<false>),
                        hipFuncAttributeMaxDynamicSharedMemorySize, kMfmaLds);
    attr_done = true;
  }
  const Seg* ss = o.segs + (size_t)(g * kNumFam + kFamStream) * kSegCap;
  int32_t* ms = o.meta + (g * kNumFam + kFamStream) * kMetaStride;
  const Seg* sm = o.segs + (size_t)(g * kNumFam + kFamMfma) * kSegCap;
  int32_t* mm = o.meta + (g * kNumFam + kFamMfma) * kMetaStride;
  if (g == kGemmGateUp) {
    gemm_stream_bf16<true><<<num_cus * 4, 256, 0, s>>>(ss, ms);
    gemm_mfma_bf16<true><<<num_cus, 256, kMfmaLds, s>>>(sm, mm);
  } else {
    gemm_stream_bf16<false><<<num_cus * 4, 256, 0, s>>>(ss, ms);
    gemm_mfma_bf16<false><<<num_cus, 256, kMfmaLds, s>>>(sm, mm);
  }
  return hipGetLastError();
}

}  // namespace moe
