// LDS-staged MFMA tiles for block-scaled fp8 (OCP e4m3) experts heavy enough to reuse a weight tile
// over many rows (prefill-sized batches).
//
// GC-MoE (summary) runs FP8 grouped GEMMs with block scales, fused SwiGLU and requantisation.  The
// weight-streaming fp8 tiles (gemm_fp8.hip) re-read an expert's weights once per 32 rows; here a
// workgroup stages a 256-row token tile and a 256-row weight tile through LDS, one 128-wide K block
// (one scale block) per stage, so each weight byte is read once per 256 rows.  Per K block kb:
//   P = sum_{k in kb} q_w[n][k] * q_x[row][k]          (one 16x16x128 fp8 MFMA, exact in fp32)
//   acc[row][n] += P * (s_w[n/128][kb] * s_x[row][kb])
// with s_w the weight's 128x128 block scale and s_x the row's 1x128 activation scale -- the same
// arithmetic as the streaming tiles.
//
// Workgroup: 8 wavefronts (two per SIMD, so one hides the other's LDS and scale latency), tile =
// 256 token rows x 256 weight rows.  Wavefront w covers tokens [64 (w & 3), +64) and weight rows
// (gate/up) gate [64 (w >> 2), +64) with the matching up rows -- h columns [64 (w >> 2), +64) of the
// tile's 128 -- or (down) [128 (w >> 2), +128): 4 token blocks x 8 weight blocks of 16, 128 fp32
// accumulators per lane.
//
// Stage (66 KB, two in a ring): 512 LDS rows of 128 bytes (tokens, then weights: gate/up 128 gate
// rows and 128 up rows), 16-byte chunks XOR-swizzled by (row >> 1) & 7, then eight 256-byte scale
// regions: token scales of rows [64 r, +64) in region r < 4, the weight scales in regions 4 and 5
// (gate/up: gate, up; down: the tile's two 128-row blocks; 6 and 7 repeat region 4 so that every
// wavefront issues the same number of loads per stage and one wait count serves all).  Every byte
// goes global -> LDS by direct loads (global_load_lds), 9 per wavefront per stage.  Weights come in
// the library's tiled fp8 layout: per 16-row block and 128-byte chunk of K, unit (h, g, r) holds
// bytes [32 g + 16 h, +16) of row r at ((h * 4 + g) * 16 + r) * 16.
//
// A lane (g = lane / 16, i = lane % 16) of a 16x16x128 MFMA operand takes row i's 32 bytes
// [32 g, 32 g + 32) -- loaded alike for both operands, so the pairing of K values inside the
// instruction does not matter (common.h).
#include "common.h"
#include "fp8_codec.h"
#include "kernels.h"
#include "mfma_dev.h"

namespace moe {

namespace {

constexpr int F8BM = kMfmaBM;                 // token rows per tile
constexpr int F8BW = 256;                     // weight rows per tile
constexpr int F8ROW = 128;                    // bytes per LDS row (one K block of e4m3)
constexpr int F8DATA = (F8BM + F8BW) * F8ROW;  // 64 KB
constexpr int F8STAGE = F8DATA + 8 * 256;     // + scale regions
constexpr int F8LOADS = 8;                    // 16-byte loads per wavefront per stage (1 KB each)
constexpr int F8VM = F8LOADS + 1;             // vector memory operations per wavefront per stage
static_assert(F8BM == 256 && kMfmaBNGateUp == 128 && kMfmaBNDown == 256, "tile geometry");
static_assert(F8DATA / 1024 == 8 * F8LOADS, "one kilobyte per load instruction");

__shared__ __attribute__((aligned(1024))) uint8_t f8_ring[2 * F8STAGE];

__device__ __forceinline__ void f8_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 32 bytes of an MFMA operand from LDS: row base (multiple of 16 rows), lane offsets of the two
// 16-byte chunks (swizzle included)
__device__ __forceinline__ i32x8 lds_frag(const uint8_t* rowbase, int o0, int o1) {
  const uint4 lo = *reinterpret_cast<const uint4*>(rowbase + o0);
  const uint4 hi = *reinterpret_cast<const uint4*>(rowbase + o1);
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// LDS row (tile-relative weight row) of weight block a (16 rows) of wavefront column wn
template <bool GU>
__device__ __forceinline__ constexpr int wblk_row(int a, int wn) {
  return GU ? (a < 4 ? 64 * wn + 16 * a : 128 + 64 * wn + 16 * (a - 4)) : 128 * wn + 16 * a;
}

template <bool GU>
struct Fp8Tile {
  // Load slot j (instruction j of the wavefront's 8 per stage) fills LDS rows [8 q, 8 q + 8),
  // q = w + 8 j: slots 0..3 token rows, 4..7 weight rows in groups of 64 (gate/up: gate rows
  // [0, 64), [64, 128), then the same up rows; down: rows 64 (j - 4) ...).  A lane's row within
  // the slot is r = lane / 8 and its chunk p = lane % 8 holds logical chunk p ^ ((8 q + r) / 2 % 8),
  // the same for every slot (q is odd exactly when w is).  Weight slots differ only by a uniform
  // byte offset, so one lane offset serves all four.
  const char* wbase[4];  // weight slot bases (uniform)
  uint32_t toff[4];      // token slots: the lane's byte offset at K block 0 (gathered rows)
  uint32_t woff;         // weight slots: the lane's byte offset in its 64-row group at K block 0
  const char* sbase;     // scale load: token scales or a weight scale
  uint32_t soff;
  const char* abase;
  f32x4 acc[8][4];       // [weight block][token block]

  __device__ __forceinline__ void setup(const Seg& sg, int m0, int rows, int n0) {
    const int lane = tid_here() & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = sg.K, nkb = K / 128;
    const int r = lane >> 3, p = lane & 7;
    const int c = p ^ ((4 * (w & 1) + (r >> 1)) & 7);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = 8 * w + 64 * j + r;   // token row of slot j
      const int rr = R < rows ? R : 0;    // padded rows re-read the first row; never stored
      const int gr = sg.row0 + m0 + rr;
      const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
      toff[j] = (uint32_t)src * (uint32_t)K + c * 16;
    }
    abase = static_cast<const char*>(sg.a);
    // weight row of slot 4 (the tiled layout: 16-row blocks of nkb 2 KB chunk units)
    const int n = n0 + 8 * w + r;
    woff = (uint32_t)(n >> 4) * (uint32_t)(nkb * 2048) +
           (uint32_t)(((c & 1) * 4 + (c >> 1)) * 256 + (n & 15) * 16);
    const size_t grp = (size_t)4 * nkb * 2048;  // 64 weight rows
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (GU) {
        wbase[j] = static_cast<const char*>(j < 2 ? sg.w0 : sg.w1) + (j & 1) * grp;
      } else {
        // (a 64-row group past N -- the edge tile of a d that is not a multiple of 256 -- re-reads
        // the first group; its results are never stored)
        wbase[j] = static_cast<const char*>(sg.w0) + (n0 + 64 * j < sg.N ? j * grp : 0);
      }
    }
    if (w < 4) {  // token scales of rows [64 w, +64)
      const int R = 64 * w + lane;
      const int rr = R < rows ? R : 0;
      const int gr = sg.row0 + m0 + rr;
      const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
      sbase = reinterpret_cast<const char*>(sg.as);
      soff = (uint32_t)src * (uint32_t)nkb * 4;
    } else {
      const int nb = n0 / 128, nbl = sg.N / 128 - 1;
      const int nb1 = GU ? nb : min(nb + 1, nbl);
      const bool second = w == 5;
      sbase = reinterpret_cast<const char*>(GU && second ? sg.s1 : sg.s0);
      soff = (uint32_t)((second ? nb1 : nb) * nkb) * 4;
    }
  }

  __device__ __forceinline__ void issue(int S, int kb) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t* st = f8_ring + S * F8STAGE;
    // (the scale load first: the compiler waits for the row gathers its offset depends on before
    // it, and such a wait placed after the other loads would also wait for all of them)
    dma4(sbase + (size_t)kb * 4, soff, (lds_void*)(st + F8DATA + w * 256));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(abase + (size_t)kb * 128, toff[j], (lds_void*)(st + (w + 8 * j) * 1024));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(wbase[j] + (size_t)kb * 2048, woff, (lds_void*)(st + (w + 8 * (j + 4)) * 1024));
  }

  __device__ __forceinline__ void compute(int S) {
    const uint8_t* st = f8_ring + S * F8STAGE;
    const uint32_t tid = tid_here();
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int wm = w & 3, wn = w >> 2;
    const int g = lane >> 4, i = lane & 15;
    const int sw = (i >> 1) & 7;
    const int o0 = i * F8ROW + (((2 * g) ^ sw) << 4);
    const int o1 = i * F8ROW + (((2 * g + 1) ^ sw) << 4);
    const float* scl = reinterpret_cast<const float*>(st + F8DATA);
    float sx[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) sx[b] = scl[wm * 64 + 16 * b + i];
    const float swa = scl[4 * 64];                       // gate, or the wavefront's first block
    const float swb = scl[5 * 64];                       // up, or the tile's second block
    const float sw0 = GU ? swa : (wn == 0 ? swa : swb);  // down: one block per wavefront
    float cA[4], cB[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      cA[b] = sw0 * sx[b];
      cB[b] = swb * sx[b];
    }
    i32x8 xb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) xb[b] = lds_frag(st + (wm * 64 + 16 * b) * F8ROW, o0, o1);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    // one weight block at a time (its next block's fragment read ahead), so that only one block's
    // products are live beside the 128 accumulators
    i32x8 wa = lds_frag(st + (F8BM + wblk_row<GU>(0, wn)) * F8ROW, o0, o1);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      i32x8 wn_next;
      if (a < 7) wn_next = lds_frag(st + (F8BM + wblk_row<GU>(a + 1, wn)) * F8ROW, o0, o1);
      f32x4 p[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) p[b] = mfma16_fp8(wa, xb[b], zero);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float c = (GU && a >= 4) ? cB[b] : cA[b];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[a][b][r] = fmaf(p[b][r], c, acc[a][b][r]);
      }
      if (a < 7) wa = wn_next;
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // nkb K blocks; two stages in a ring, the next block's loads in flight while one is computed
  __device__ __forceinline__ void run(int nkb) {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    if (nkb > 1) issue(1, 1);
    for (int kb = 0; kb < nkb; ++kb) {
      const int S = kb & 1;
      if (kb + 1 < nkb) MOE_WAITCNT(F8VM, 15);
      else MOE_WAITCNT(0, 15);
      f8_barrier();
      compute(S);
      MOE_WAITCNT(63, 0);
      f8_barrier();
      if (kb + 2 < nkb) issue(S, kb + 2);
    }
  }
};

// Gate/up epilogue: h = SiLU(g) * u for the tile's 128 columns, requantised per token row over
// them (one 128-wide scale block: s = amax / 448, q = e4m3(h * (1 / s)), as the streaming tiles),
// e4m3 h and its scale stored.  red: 2 x 256 floats of LDS (per-wavefront-column row maxima).
__device__ __forceinline__ void f8_gateup_store(const f32x4 (&acc)[8][4], const Seg& sg, int m0,
                                                int rows, int n0, float* red) {
  const uint32_t tid = tid_here();
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w & 3, wn = w >> 2;
  const int g = lane >> 4, i = lane & 15;
  float h[4][4][4];  // [gate block a][token block b][r]
  float amax[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    amax[b] = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        h[a][b][r] = swiglu(acc[a][b][r], acc[a + 4][b][r]);
        amax[b] = fmaxf(amax[b], fabsf(h[a][b][r]));
      }
    amax[b] = fmaxf(amax[b], __shfl_xor(amax[b], 16));
    amax[b] = fmaxf(amax[b], __shfl_xor(amax[b], 32));
  }
  f8_barrier();  // the previous tile's readers of red[] are done
  if (g == 0) {
#pragma unroll
    for (int b = 0; b < 4; ++b) red[wn * 256 + wm * 64 + 16 * b + i] = amax[b];
  }
  MOE_WAITCNT(63, 0);
  f8_barrier();
  const int N = sg.N;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int t = wm * 64 + 16 * b + i;
    const float m = fmaxf(red[t], red[256 + t]);
    float s = m / 448.0f;
    if (m == 0.0f || s == 0.0f) s = 1.0f;
    const float inv = 1.0f / s;
    if (t < rows) {
      const size_t orow = (size_t)(sg.row0 + m0 + t);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint32_t pk = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) pk |= uint32_t(e4m3_encode(h[a][b][r] * inv)) << (8 * r);
        gstore4(sg.out, orow * N + n0 + 64 * wn + 16 * a + 4 * g, pk);
      }
      if (wn == 0 && g == 0) gstore_f32(sg.outs, orow * (N / 128) + n0 / 128, s);
    }
  }
}

// Down epilogue: bf16 y for the wavefront's 128 columns (none past N).
__device__ __forceinline__ void f8_down_store(const f32x4 (&acc)[8][4], const Seg& sg, int m0,
                                              int rows, int n0) {
  const uint32_t tid = tid_here();
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w & 3, wn = w >> 2;
  const int g = lane >> 4, i = lane & 15;
  const int N = sg.N;
  if (n0 + 128 * wn >= N) return;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int t = wm * 64 + 16 * b + i;
    if (t >= rows) continue;
    const size_t orow = (size_t)(sg.row0 + m0 + t) * N;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      uint2 pk;
      pk.x = pack_bf16x2(acc[a][b][0], acc[a][b][1]);
      pk.y = pack_bf16x2(acc[a][b][2], acc[a][b][3]);
      gstore8(sg.out, (orow + n0 + 128 * wn + 16 * a + 4 * g) * 2, pk);
    }
  }
}

// Persistent: one workgroup per CU takes tiles from the per-XCD queues (tile order: heavy experts'
// tiles with the light ones spread between them, as the bf16 MFMA lists in their mixed order).
template <bool GU>
__global__ __launch_bounds__(512, 1) void gemm_mfma_fp8(const Seg* __restrict__ segs,
                                                         int32_t* __restrict__ meta) {
  __shared__ int slot;
  __shared__ int seg_base[kSegCap];
  __shared__ float red[2 * 256];
  const int ntiles = meta[1];
  if (ntiles == 0) return;
  const int nseg = meta[0], ntiles0 = meta[kMetaClass0];
  const int chunk = max(1, (int)gridDim.x / kXcds);
  for (int i = threadIdx.x; i < nseg; i += blockDim.x) seg_base[i] = segs[i].tile_base;
  __syncthreads();
  Fp8Tile<GU> tile;
  int q = 0;
  for (;;) {
    // (the counts go through an opaque move each tile: otherwise the reciprocals of the queue's
    // integer divisions are hoisted out of the loop and held, or spilled, across the K loop)
    const int nt_ = opaque_s(ntiles), ch_ = opaque_s(chunk), nt0_ = opaque_s(ntiles0);
    const int pos = pop_tile_xcd(meta + kMetaQueue, nt_, ch_, &slot, q);
    if (pos < 0) break;
    const int t = interleave_tile(pos, nt0_, nt_);
    const Seg& sg = segs[__builtin_amdgcn_readfirstlane(find_seg_lds(seg_base, nseg, t))];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * F8BM;
    const int rows = min(F8BM, sg.rows - m0);
    const int n0 = nt * (GU ? kMfmaBNGateUp : kMfmaBNDown);
    tile.setup(sg, m0, rows, n0);
    tile.run(sg.K / 128);
    if (GU) f8_gateup_store(tile.acc, sg, m0, rows, n0, red);
    else f8_down_store(tile.acc, sg, m0, rows, n0);
  }
}

}  // namespace

void launch_mfma_fp8(const Seg* segs, int32_t* meta, int gemm, int num_cus, hipStream_t s) {
  if (gemm == kGemmGateUp) gemm_mfma_fp8<true><<<num_cus, 512, 0, s>>>(segs, meta);
  else gemm_mfma_fp8<false><<<num_cus, 512, 0, s>>>(segs, meta);
}

}  // namespace moe
