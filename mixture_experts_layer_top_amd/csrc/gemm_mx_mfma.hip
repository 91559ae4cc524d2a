// LDS-staged MFMA tiles for MXFP4 experts with MXFP8 activations, for experts heavy enough to reuse
// a weight tile over many rows (prefill-sized batches).
//
// GC-MoE (summary) runs FP4 grouped GEMMs as block-scaled matrix multiplies.  The streaming MX tiles
// (gemm_mx.hip) re-read an expert's weights once per 32 rows; here a workgroup stages a 256-row
// token tile and a 256-row weight tile through LDS, one 128-wide K chunk per stage, so each weight
// byte is read once per 256 rows.  v_mfma_scale_f32_16x16x128_f8f6f4 applies both operands' E8M0
// scales itself (weights format 4 = E2M1, activations format 0 = E4M3), so the accumulators take the
// scaled products directly: no per-block arithmetic outside the matrix unit.
//
// Workgroup: 8 wavefronts (two per SIMD), tile = 256 token rows x 256 weight rows; wavefront w covers
// tokens [64 (w & 3), +64) and weight rows (gate/up) gate [64 (w >> 2), +64) with the matching up
// rows, or (down) [128 (w >> 2), +128): 4 token blocks x 8 weight blocks of 16.
//
// Operand layout (a lane-layout probe of the instruction; lane l = 16 g + i holds row i):
//   E2M1 weights (16 bytes): K values 32 g .. 32 g + 31 -- exactly unit (g, i) of the library's
//     tiled MXFP4 layout (per 16-row block and 128-value chunk, 1 KB ordered [g][row][16 bytes]),
//     so a weight block is one 1 KB copy into LDS and one ds_read_b128 per lane;
//   E4M3 activations (32 bytes): K values 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15 of the
//     row (16-byte chunks g and 4 + g of its 128 bytes);
//   scales: lane 16 b + i carries row i's E8M0 byte of K block b (values 32 b .. 32 b + 31).
//
// Stage (50 KB, two in a ring): 256 token rows of 128 bytes (16-byte chunks XOR-swizzled by
// (row >> 1) & 7), 16 weight blocks of 1 KB (gate/up: 8 gate blocks, then 8 up blocks), the 256
// weight rows' 4 scale bytes of the chunk, the 256 token rows' 4 scale bytes.  Everything goes
// global -> LDS by direct loads, 7 per wavefront per stage (4 token, 2 weight, 1 scale), so one
// explicit vmcnt serves every wavefront.
#include "common.h"
#include "fp8_codec.h"
#include "kernels.h"
#include "mfma_dev.h"
#include "mx_codec.h"

namespace moe {

namespace {

constexpr int XBM = kMfmaBM;                   // token rows per tile
constexpr int XBW = 256;                       // weight rows per tile
constexpr int XTOK = XBM * 128;                // token bytes per stage (32 KB)
constexpr int XWGT = XBW / 16 * 1024;          // weight bytes per stage (16 KB)
constexpr int XWSC = XTOK + XWGT;              // weight scales: 4 bytes per weight row
constexpr int XTSC = XWSC + XBW * 4;           // token scales: 4 bytes per token row
constexpr int XSTAGE = XTSC + XBM * 4;         // 50 KB
constexpr int XVM = 7;                         // vector memory operations per wavefront per stage
static_assert(XBM == 256 && kMfmaBNGateUp == 128 && kMfmaBNDown == 256, "tile geometry");
static_assert(XTOK / 1024 == 4 * 8 && XWGT / 1024 == 2 * 8, "load slots");

__shared__ __attribute__((aligned(1024))) uint8_t mx_ring[2 * XSTAGE];

__device__ __forceinline__ void mx_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma_mx4(const i32x4& w, uint32_t sw, const i32x8& x, uint32_t sx,
                                          const f32x4& c) {
  // A: E2M1 (format 4, only the first four dwords are read); B: E4M3 (format 0)
  const i32x8 a = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, x, c, 4, 0, 0, (int)sw, 0, (int)sx);
}

// LDS row (tile-relative weight row) of weight block a (16 rows) of wavefront column wn
template <bool GU>
__device__ __forceinline__ constexpr int xblk_row(int a, int wn) {
  return GU ? (a < 4 ? 64 * wn + 16 * a : 128 + 64 * wn + 16 * (a - 4)) : 128 * wn + 16 * a;
}

template <bool GU>
struct MxTile {
  // Load slots of wavefront w: token instructions w + 8 j (j < 4; LDS token rows [8 q, 8 q + 8) of
  // q = w + 8 j), weight blocks w + 8 j (j < 2), and one scale instruction: w < 4 the weight
  // scales of rows [64 w, +64), else the token scales of rows [64 (w - 4), +64).
  uint32_t toff[4];     // token slots: the lane's byte offset at chunk 0 (gathered rows)
  const char* abase;
  const char* wbase[2];  // weight blocks of the two slots (uniform), at chunk 0
  const char* sbase;     // the scale instruction's base
  uint32_t soff;         // its lane offset at chunk 0
  uint32_t wstride;      // bytes per chunk of a weight block (1 KB) and of a scale row (4)
  f32x4 acc[8][4];       // [weight block][token block]

  __device__ __forceinline__ void setup(const Seg& sg, int m0, int rows, int n0) {
    const int lane = tid_here() & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int K = sg.K, nch = K / 128, KB = K / 32;
    const int r = lane >> 3, p = lane & 7;
    const int c = p ^ ((4 * (w & 1) + (r >> 1)) & 7);  // (the same for every token slot)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = 8 * w + 64 * j + r;
      const int rr = R < rows ? R : 0;  // padded rows re-read the first row; never stored
      const int gr = sg.row0 + m0 + rr;
      const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
      toff[j] = (uint32_t)src * (uint32_t)K + c * 16;
    }
    abase = static_cast<const char*>(sg.a);
    // weight block slot j: tile block bb = w + 8 j (gate/up: 0..7 gate, 8..15 up)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int bb = w + 8 * j;
      int row = GU ? n0 + 16 * (bb & 7) : n0 + 16 * bb;
      row = row < sg.N ? row : sg.N - 16;  // (down: the edge tile's blocks past N re-read the last)
      const char* base = static_cast<const char*>(GU && bb >= 8 ? sg.w1 : sg.w0);
      wbase[j] = base + (size_t)(row >> 4) * nch * 1024;
    }
    if (w < 4) {  // weight scales of tile rows [64 w, +64): 4 bytes of the chunk per row
      const int tr = 64 * w + lane;
      int row = GU ? n0 + (tr & 127) : n0 + tr;
      row = row < sg.N ? row : sg.N - 1;
      sbase = reinterpret_cast<const char*>(GU && tr >= 128 ? sg.e1 : sg.e0);
      soff = (uint32_t)row * (uint32_t)KB;
    } else {  // token scales of rows [64 (w - 4), +64)
      const int R = 64 * (w - 4) + lane;
      const int rr = R < rows ? R : 0;
      const int gr = sg.row0 + m0 + rr;
      const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
      sbase = reinterpret_cast<const char*>(sg.ae);
      soff = (uint32_t)src * (uint32_t)KB;
    }
  }

  __device__ __forceinline__ void issue(int S, int ch) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint8_t* st = mx_ring + S * XSTAGE;
    // (the scale load first: the compiler waits for the row gathers its offset depends on before
    // it, and such a wait placed after the other loads would also wait for all of them)
    dma4(sbase + (size_t)ch * 4, soff,
         (lds_void*)(st + (w < 4 ? XWSC + 256 * w : XTSC + 256 * (w - 4))));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(abase + (size_t)ch * 128, toff[j], (lds_void*)(st + (w + 8 * j) * 1024));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      dma16(wbase[j] + (size_t)ch * 1024, (uint32_t)lane * 16,
            (lds_void*)(st + XTOK + (w + 8 * j) * 1024));
  }

  __device__ __forceinline__ void compute(int S) {
    const uint8_t* st = mx_ring + S * XSTAGE;
    const uint32_t tid = tid_here();
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int wm = w & 3, wn = w >> 2;
    const int g = lane >> 4, i = lane & 15;
    const int sw = (i >> 1) & 7;
    const int o0 = i * 128 + ((g ^ sw) << 4);        // token chunk g
    const int o1 = i * 128 + (((4 + g) ^ sw) << 4);  // token chunk 4 + g
    i32x8 xb[4];
    uint32_t sx[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint8_t* rb = st + (wm * 64 + 16 * b) * 128;
      const uint4 lo = *reinterpret_cast<const uint4*>(rb + o0);
      const uint4 hi = *reinterpret_cast<const uint4*>(rb + o1);
      xb[b] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sx[b] = st[XTSC + (wm * 64 + 16 * b + i) * 4 + g];
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int wr = xblk_row<GU>(a, wn);  // tile weight row of the block (a multiple of 16)
      const uint4 v = *reinterpret_cast<const uint4*>(st + XTOK + (wr >> 4) * 1024 + lane * 16);
      const i32x4 wa = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      const uint32_t swa = st[XWSC + (wr + i) * 4 + g];
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma_mx4(wa, swa, xb[b], sx[b], acc[a][b]);
    }
  }

  // nch K chunks; two stages in a ring, the next chunk's loads in flight while one is computed
  __device__ __forceinline__ void run(int nch) {
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    if (nch > 1) issue(1, 1);
    for (int ch = 0; ch < nch; ++ch) {
      const int S = ch & 1;
      if (ch + 1 < nch) MOE_WAITCNT(XVM, 15);
      else MOE_WAITCNT(0, 15);
      mx_barrier();
      compute(S);
      MOE_WAITCNT(63, 0);  // this wavefront's reads of stage S are done
      mx_barrier();
      if (ch + 2 < nch) issue(S, ch + 2);
    }
  }
};

// Gate/up epilogue: h = SiLU(g) * u for the wavefront's 64 columns, requantised to MXFP8 per token
// row and 32 columns (two weight blocks, all in this wavefront: a max over the lane's 8 values and
// the 4 lane groups), e4m3 h and its E8M0 scales stored.
__device__ __forceinline__ void mx_mfma_gateup_store(const f32x4 (&acc)[8][4], const Seg& sg, int m0,
                                                     int rows, int n0) {
  const uint32_t tid = tid_here();
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w & 3, wn = w >> 2;
  const int g = lane >> 4, i = lane & 15;
  const int N = sg.N;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int t = wm * 64 + 16 * b + i;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {  // 32-column block: gate blocks 2 hb, 2 hb + 1
      float h[2][4];
      float amax = 0.f;
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          h[s][r] = swiglu(acc[2 * hb + s][b][r], acc[4 + 2 * hb + s][b][r]);
          amax = fmaxf(amax, fabsf(h[s][r]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const int X = mx_scale_code(amax);
      const float inv = mx_inv_scale(X);
      if (t < rows) {
        const size_t orow = (size_t)(sg.row0 + m0 + t);
        const int c0 = n0 + 64 * wn + 32 * hb;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint32_t pk = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) pk |= uint32_t(e4m3_encode(h[s][r] * inv)) << (8 * r);
          gstore4(sg.out, orow * N + c0 + 16 * s + 4 * g, pk);
        }
        if (g == 0) gstore_u8(sg.oute, orow * (N / 32) + c0 / 32, uint32_t(X));
      }
    }
  }
}

// Down epilogue: bf16 y for the wavefront's 128 columns (none past N).
__device__ __forceinline__ void mx_mfma_down_store(const f32x4 (&acc)[8][4], const Seg& sg, int m0,
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

// Persistent: one workgroup per CU takes tiles from the per-XCD queues (mixed tile order).
template <bool GU>
__global__ __launch_bounds__(512, 1) void gemm_mfma_mx(const Seg* __restrict__ segs,
                                                       int32_t* __restrict__ meta) {
  __shared__ int slot;
  __shared__ int seg_base[kSegCap];
  const int ntiles = meta[1];
  if (ntiles == 0) return;
  const int nseg = meta[0], ntiles0 = meta[kMetaClass0];
  const int chunk = max(1, (int)gridDim.x / kXcds);
  for (int i = threadIdx.x; i < nseg; i += blockDim.x) seg_base[i] = segs[i].tile_base;
  __syncthreads();
  MxTile<GU> tile;
  int q = 0;
  for (;;) {
    // (the counts go through an opaque move each tile: otherwise the reciprocals of the queue's
    // integer divisions are hoisted out of the loop and held across the K loop)
    const int nt_ = opaque_s(ntiles), ch_ = opaque_s(chunk), nt0_ = opaque_s(ntiles0);
    const int pos = pop_tile_xcd(meta + kMetaQueue, nt_, ch_, &slot, q);
    if (pos < 0) break;
    const int t = interleave_tile(pos, nt0_, nt_);
    const Seg& sg = segs[__builtin_amdgcn_readfirstlane(find_seg_lds(seg_base, nseg, t))];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * XBM;
    const int rows = min(XBM, sg.rows - m0);
    const int n0 = nt * (GU ? kMfmaBNGateUp : kMfmaBNDown);
    tile.setup(sg, m0, rows, n0);
    tile.run(sg.K / 128);
    if (GU) mx_mfma_gateup_store(tile.acc, sg, m0, rows, n0);
    else mx_mfma_down_store(tile.acc, sg, m0, rows, n0);
  }
}

}  // namespace

void launch_mfma_mx(const Seg* segs, int32_t* meta, int gemm, int num_cus, hipStream_t s) {
  if (gemm == kGemmGateUp) gemm_mfma_mx<true><<<num_cus, 512, 0, s>>>(segs, meta);
  else gemm_mfma_mx<false><<<num_cus, 512, 0, s>>>(segs, meta);
}

}  // namespace moe
