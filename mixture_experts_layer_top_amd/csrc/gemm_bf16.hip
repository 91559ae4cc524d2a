// Grouped expert GEMMs, bf16 weights and activations, fp32 accumulation on MFMA.
//
// Gate/up: h[row][n] = SiLU(sum_k x[tok(row)][k] Wg[n][k]) * (sum_k x[tok(row)][k] Wu[n][k]),
// with the token gather fused into the activation loads (GC-MoE, summary: grouped GEMM with fused
// SwiGLU).  Down: y[row][n] = sum_k h[row][k] Wd[n][k].  Shapes follow the live routing histogram
// ("Decoding the Skew ...", Abstract: sparse expert GEMMs whose shapes vary with routing).
//
// Two tile families, chosen per expert and GEMM on the device (select.hip):
//  * stream: one workgroup = 4 wavefronts x 16 weight rows (or 16 each), up to 64 of an expert's
//    rows per pass.  Operand roles are swapped so the weight rows sit on the MFMA's 16-wide row
//    side and the few tokens on the column side (the same idea as GC-MoE's operand-swapped MMA);
//    weights go straight from HBM into MFMA registers, each element used once, 64 contiguous bytes
//    per row per load.
//  * mfma: 256 token rows x 256 weight rows per tile, K-steps of 64 staged through two LDS stages
//    by direct global->LDS loads with an XOR swizzle (conflict-free ds_read_b128), 2x2 wavefronts
//    of 128x128, MFMA 32x32x16.
// Both are persistent: a fixed grid pops tiles from device queues (zeroed by the selection
// kernel), heaviest experts first, m-tiles of one weight tile adjacent in the queue.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "route_dev.h"
#include "mfma_dev.h"
#include "stream_dev.h"

namespace moe {

// XL > 0: the tile has one row, whose activations (K bf16) the MFMA loop reads from LDS (xs): with
// XL = 1 the tile stages them from xrow once its first weight loads are in flight, with XL = 2 the
// caller has staged them.
template <int MQ, bool GU, int WK, int XL = 0, bool COH = false>
__device__ __forceinline__ void stream_tile_bf16(const Seg& sg, int m0, int rows, int n0,
                                                 float* red, const char* xs = nullptr,
                                                 const void* xrow = nullptr) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = sg.K;
  // WK wavefronts split K over each group of 16 weight rows; the 4 / WK groups are consecutive
  const int grp = wv / WK, kw = wv % WK;
  n0 += 16 * grp;
  const int nrow = n0 + r16;  // this lane's weight row (A operand)
  const void* wg = sg.w0;
  const void* wu = GU ? sg.w1 : sg.w0;
  const void* xa = sg.a;
  const int kq = K / WK;  // this wavefront's K range [kw*kq, (kw+1)*kq); K % 128 == 0
  const uint32_t kbase = (uint32_t)(kw * kq) * 2 + kg * 16;
  const uint32_t woff = (uint32_t)nrow * K * 2 + kbase;
  uint32_t xoff[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;  // padded columns re-read a valid row; never stored
    const int gr = sg.row0 + m0 + r;
    const int src = XL ? 0 : sg.tok ? gload_i32(sg.tok, gr) : gr;
    xoff[q] = (uint32_t)src * K * 2 + kbase;  // (XL: byte offset in the staged row)
  }
  f32x4 acc0[MQ], acc1[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    acc0[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr int U = (MQ == 1) ? 4 : 2;  // K-steps (of 32) per batch
  struct Batch { uint4 a0[U], a1[U], b[U][MQ]; };
  auto load = [&](Batch& bt, int ks) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t ko = (uint32_t)(ks + u) * 64;
      bt.a0[u] = gload16(wg, woff + ko);
      if (GU) bt.a1[u] = gload16(wu, woff + ko);
      if (!XL) {
#pragma unroll
        for (int q = 0; q < MQ; ++q) bt.b[u][q] = gload16(xa, xoff[q] + ko);
      }
    }
  };
  auto xfrag = [&](const Batch& bt, int u, int q, int ks) {
    return XL ? *reinterpret_cast<const uint4*>(xs + xoff[q] + (uint32_t)(ks + u) * 64)
              : bt.b[u][q];
  };
  auto compute = [&](const Batch& bt, int ks) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        const uint4 b = xfrag(bt, u, q, ks);
        acc0[q] = mfma16(as_bf16x8(bt.a0[u]), as_bf16x8(b), acc0[q]);
        if (GU) acc1[q] = mfma16(as_bf16x8(bt.a1[u]), as_bf16x8(b), acc1[q]);
      }
  };
  const int nsteps = kq / 32;             // K-steps of this wavefront (>= 1)
  const int nfull = nsteps / U * U;        // pipelined part: whole batches only
  // (Pinning the load groups with scheduling barriers and branch-free loads, as the MXFP4 tiles
  // do, measured neutral here -- DeepSeek-V3-shaped decode within 1%, the down GEMM up to 2.5%
  // slower at T = 64: four wavefronts per SIMD cover the drained waits.)
  Batch b0, b1;
  if (nfull > 0) load(b0, 0);
  if (XL == 1) {
    // stage the row's activations (the first weight loads are already in flight); the previous
    // tile's readers of xs all passed the barrier before its split-K reduction
    const uint4* xg = static_cast<const uint4*>(xrow);
    uint4* xw = reinterpret_cast<uint4*>(const_cast<char*>(xs));
    for (int i = threadIdx.x; i < K / 8; i += 256) xw[i] = xg[i];
    __syncthreads();
  }
  for (int ks = 0; ks < nfull; ks += 2 * U) {
    if (ks + U < nfull) load(b1, ks + U);
    compute(b0, ks);
    if (ks + 2 * U < nfull) load(b0, ks + 2 * U);
    if (ks + U < nfull) compute(b1, ks + U);
  }
  for (int ks = nfull; ks < nsteps; ++ks) {  // remainder, one K-step at a time
    const uint32_t ko = (uint32_t)ks * 64;
    const uint4 a0 = gload16(wg, woff + ko);
    const uint4 a1 = GU ? gload16(wu, woff + ko) : a0;
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const uint4 b = XL ? *reinterpret_cast<const uint4*>(xs + xoff[q] + ko) : gload16(xa, xoff[q] + ko);
      acc0[q] = mfma16(as_bf16x8(a0), as_bf16x8(b), acc0[q]);
      if (GU) acc1[q] = mfma16(as_bf16x8(a1), as_bf16x8(b), acc1[q]);
    }
  }
  stream_tile_finish<MQ, GU, WK, COH>(sg, m0, rows, n0, red, acc0, acc1);
}

// MXFP4 weights (W4A16), in the library's tiled layout (moe_mxfp4_tile): per 16-row block and
// 128-value chunk of K, 1 KB ordered [lane group kg][row r][16 bytes = values 32 kg .. 32 kg + 31
// of the chunk], so lane kg * 16 + r of a wavefront reads bytes [16 lane, +16) of the chunk and one
// load instruction reads 1 KB contiguously; E8M0 scales stay row-major [N][K/32].  The
// MFMA operands are the bf16 values e2m1 * 2^(X - 127), converted in registers (the scaled fp4 ->
// bf16 conversion, two per instruction; exact, since every such product is a bf16 value), so the
// tile is the bf16 streaming tile with a quarter of the weight bytes.  Inside a batch of U K-steps
// each lane takes U/4 pieces of 32 consecutive K values (piece i: chunk 2 c + i for U = 8, 8 values
// per step), so its weights are U/4 16-byte loads from the tiled layout and its scales whole blocks
// of 32; U = 8 for one token group keeps as many bytes in flight
// per CU as the bf16 tile's four steps.  A step's K values per lane only have to agree between the
// two operands, so the order differs from the bf16 tile's.  Leftover steps run one at a time.
// Each wavefront group covers NR = 2 sets of 16 weight rows against the same activation fragments
// (the tile is twice the bf16 tile's width): activations are bf16, four times the bytes of the
// weights per K, and they are re-read from L2 once per 16 weight rows.  The WK wavefronts of a
// group take interleaved chunks of 32*U K values (chunk c goes to wavefront c % WK), so at any
// time they read adjacent bytes of each weight row (longer DRAM runs than contiguous quarters of
// K: gate/up 4% faster); what is left after whole rounds of chunks is split contiguously.
__device__ __forceinline__ uint4 decode_e2m1x8(uint32_t packed, uint32_t scale_code) {
  const float sc = __builtin_bit_cast(float, scale_code << 23);  // 2^(X - 127), X >= 1
  uint4 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 0));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 1));
  r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 2));
  r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 3));
  return r;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Stages the E8M0 scales of the workgroup's wrows weight rows from n0 (gate, then up) into LDS (sc),
// KB bytes each at a row stride of w4_scale_stride(KB) bytes, by direct global->LDS loads (a dword
// per lane, 256 bytes per instruction; lanes past the row re-read its last dword into the
// padding).  Read per batch and lane from global memory instead, each scale load touched 16 rows'
// cache lines.  The caller waits for the loads (vmcnt(0)) and holds a barrier before reading; the
// previous pass's reads of sc are behind the barriers of its split-K reduction.
__device__ __forceinline__ int w4_scale_stride(int KB) { return (KB + 255) & ~255; }

template <bool GU>
__device__ __forceinline__ void stage_scales_w4(const Seg& sg, int n0, int wrows, int KB,
                                                uint8_t* sc) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KW = KB / 4, RS = w4_scale_stride(KB);
  const int nrow = (GU ? 2 : 1) * wrows;
  for (int r = wv; r < nrow; r += 4) {
    const uint8_t* base = GU && r >= wrows ? sg.e1 : sg.e0;
    const uint32_t row = (uint32_t)(n0 + (r < wrows ? r : r - wrows));
    for (int i = 0; i < RS / 256; ++i) {
      const int c = min(64 * i + lane, KW - 1);
      dma4(reinterpret_cast<const char*>(base), row * (uint32_t)KB + 4 * c,
           (lds_void*)(sc + r * RS + 256 * i));
    }
  }
}

template <int MQ, bool GU, int WK>
__device__ __forceinline__ void stream_tile_w4(const Seg& sg, int m0, int rows, int n0, float* red,
                                               uint8_t* sc) {
  constexpr int NR = 2;  // sets of 16 weight rows per wavefront group
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = sg.K, KB = K / 32, RS = w4_scale_stride(KB);
  const int grp = wv / WK, kw = wv % WK;
  const int wrows = 16 * NR * (4 / WK);  // weight rows of the workgroup
  const int n0wg = n0;
  n0 += 16 * NR * grp;
  uint32_t wblk[NR], srow[NR];  // byte offsets of each 16-row block; this lane's scale rows in LDS
#pragma unroll
  for (int h = 0; h < NR; ++h) {
    wblk[h] = (uint32_t)(n0 + 16 * h) * (uint32_t)(K / 2);
    srow[h] = (uint32_t)(16 * NR * grp + 16 * h + r16) * (uint32_t)RS;
  }
  const uint32_t srow1 = (uint32_t)(wrows * RS);  // the up matrix's scales follow the gate's
  uint32_t xrow[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;  // padded columns re-read a valid row; never stored
    const int gr = sg.row0 + m0 + r;
    const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
    xrow[q] = (uint32_t)src * K * 2;
  }
  MOE_WAITCNT(0, 15);  // (the row gathers have landed: no wait behind the staging loads later)
  stage_scales_w4<GU>(sg, n0wg, wrows, KB, sc);
  f32x4 acc0[NR][MQ], acc1[NR][MQ];
#pragma unroll
  for (int h = 0; h < NR; ++h)
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      acc0[h][q] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[h][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  constexpr int U = (MQ == 1) ? 8 : 4;  // K-steps (of 32) per batch
  constexpr int NW = U / 4;              // 16-byte weight loads (32 values, one scale) per batch
  struct Batch { uint4 w0[NR][NW], w1[NR][NW]; uint4 b[U][MQ]; uint32_t c0; };
  constexpr int CK = 32 * U;             // K of one batch of the 4 lane groups (a chunk)
  const int nchunk = K / CK / WK;        // chunks per wavefront: chunk c = j * WK + kw (interleaved)
  const int kr0 = nchunk * WK * CK;      // remainder [kr0, K), split contiguously
  const int rsteps = (K - kr0) / 32 / WK;
  const int kr = kr0 + kw * rsteps * 32;
  auto load = [&](Batch& bt, int j) {
    const uint32_t c0 = (uint32_t)(j * WK + kw) * NW;  // first 128-value chunk of this batch
    bt.c0 = c0;
#pragma unroll
    for (int h = 0; h < NR; ++h)
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t wo = wblk[h] + (c0 + i) * 1024 + lane * 16;
        // gate/up: whole 1 KB units of the tiled layout, read once, with the non-temporal policy
        // (gate/up -7 to -8% at T = 16 and 64); the down weights keep the default one (+2-3%)
        bt.w0[h][i] = GU ? gload16_nt(sg.w0, wo) : gload16(sg.w0, wo);
        if (GU) bt.w1[h][i] = gload16_nt(sg.w1, wo);
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // step u: piece u / 4, values 32 kg + 8 (u % 4) .. + 8 of its chunk
      const uint32_t kx = (c0 + (u >> 2)) * 128 + 32 * kg + 8 * (u & 3);
#pragma unroll
      for (int q = 0; q < MQ; ++q) bt.b[u][q] = gload16(sg.a, xrow[q] + kx * 2);
    }
  };
  auto compute = [&](const Batch& bt) {
    // the scales of the batch's pieces: block 4 (c0 + i) + kg of the lane's rows
    uint32_t s0[NR][NW], s1[NR][NW];
#pragma unroll
    for (int h = 0; h < NR; ++h)
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const uint32_t so = srow[h] + (bt.c0 + i) * 4 + kg;
        s0[h][i] = sc[so];
        if (GU) s1[h][i] = sc[srow1 + so];
      }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < NR; ++h) {
        const uint4 a0 = decode_e2m1x8(dword_of(bt.w0[h][u >> 2], u & 3), s0[h][u >> 2]);
        const uint4 a1 = GU ? decode_e2m1x8(dword_of(bt.w1[h][u >> 2], u & 3), s1[h][u >> 2]) : a0;
#pragma unroll
        for (int q = 0; q < MQ; ++q) {
          acc0[h][q] = mfma16(as_bf16x8(a0), as_bf16x8(bt.b[u][q]), acc0[h][q]);
          if (GU) acc1[h][q] = mfma16(as_bf16x8(a1), as_bf16x8(bt.b[u][q]), acc1[h][q]);
        }
      }
  };
  // Two batches in registers, the next one's loads in flight while one is computed; scheduling
  // barriers and branch-free loads (past the last batch: a re-read, never computed) keep the loads
  // where they are written (see the bf16 streaming tile).  The first batch's loads go out before
  // the wait for the staged scales.
  Batch b0, b1;
  if (nchunk > 0) load(b0, 0);
  MOE_WAITCNT(0, 0);
  __syncthreads();
  int j = 0;
  for (; j + 2 <= nchunk; j += 2) {
    load(b1, j + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(b0);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, min(j + 2, nchunk - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (j < nchunk) compute(b0);
  for (int ks = 0; ks < rsteps; ++ks) {  // remainder: lane kg takes K [32 st + 8 kg, +8)
    const uint32_t st = (uint32_t)(kr / 32 + ks);  // global 32-step: chunk st / 4, slot st % 4
    const uint32_t kl = 32 * st + 8 * kg;
    const uint32_t wo = (st >> 2) * 1024 + ((st & 3) * 16 + r16) * 16 + 4 * kg;
    uint4 b[MQ];
#pragma unroll
    for (int q = 0; q < MQ; ++q) b[q] = gload16(sg.a, xrow[q] + kl * 2);
#pragma unroll
    for (int h = 0; h < NR; ++h) {
      const uint32_t sb = srow[h] + st;
      const uint4 a0 = decode_e2m1x8(gload4(sg.w0, wblk[h] + wo), sc[sb]);
      const uint4 a1 = GU ? decode_e2m1x8(gload4(sg.w1, wblk[h] + wo), sc[srow1 + sb]) : a0;
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        acc0[h][q] = mfma16(as_bf16x8(a0), as_bf16x8(b[q]), acc0[h][q]);
        if (GU) acc1[h][q] = mfma16(as_bf16x8(a1), as_bf16x8(b[q]), acc1[h][q]);
      }
    }
  }
  // one reduction and epilogue per set of 16 rows (each ends with every wavefront past its barriers)
#pragma unroll
  for (int h = 0; h < NR; ++h)
    stream_tile_finish<MQ, GU, WK>(sg, m0, rows, n0 + 16 * h, red, acc0[h], acc1[h]);
}

// Rows [m0, m0 + rows) of one tile, in passes of at most 16 * MQMAX rows.  The kernel's register
// budget is that of its widest pass, so the host instantiates MQMAX from a bound on any expert's
// rows (every expert holds at most T rows): at MQMAX = 1 four workgroups fit on each CU.
// MQMAX = 0 (the host launches it when every expert holds at most one row, as at T = 1, and K <=
// kStreamXlMaxK): rows one at a time, each staging its activations in LDS (xs) for the MFMA loop.
template <bool GU, int WK, int MQMAX, bool W4>
__device__ __forceinline__ void stream_rows_bf16(const Seg& sg, int m0, int rows, int n0,
                                                 float* red, const char* xs, uint8_t* sc) {
  static_assert(!(W4 && MQMAX == 0), "mxfp4 tiles do not stage a row in LDS");
  if (W4) {
    constexpr int MQ = MQMAX > 0 ? MQMAX : 1;
    for (int sub = 0; sub < rows; sub += 16 * MQ) {
      const int r = min(16 * MQ, rows - sub);
      if (MQ == 1 || r <= 16) stream_tile_w4<1, GU, WK>(sg, m0 + sub, r, n0, red, sc);
      else if (MQ == 2 || r <= 32) stream_tile_w4<MQ >= 2 ? 2 : 1, GU, WK>(sg, m0 + sub, r, n0, red, sc);
      else stream_tile_w4<MQ, GU, WK>(sg, m0 + sub, r, n0, red, sc);
    }
    return;
  }
  if (MQMAX == 0) {
    if (sg.K > kStreamXlMaxK) return;  // (excluded by the host)
    for (int r = 0; r < rows; ++r) {
      const int gr = sg.row0 + m0 + r;
      const int src = sg.tok ? gload_i32(sg.tok, gr) : gr;
      const void* xrow = static_cast<const char*>(sg.a) + (size_t)src * sg.K * 2;
      stream_tile_bf16<1, GU, WK, 1>(sg, m0 + r, 1, n0, red, xs, xrow);
    }
    return;
  }
  constexpr int MQ = MQMAX > 0 ? MQMAX : 1;
  for (int sub = 0; sub < rows; sub += 16 * MQ) {
    const int r = min(16 * MQ, rows - sub);
    if (MQ == 1 || r <= 16) stream_tile_bf16<1, GU, WK>(sg, m0 + sub, r, n0, red);
    else if (MQ == 2 || r <= 32) stream_tile_bf16<MQ >= 2 ? 2 : 1, GU, WK>(sg, m0 + sub, r, n0, red);
    else stream_tile_bf16<MQ, GU, WK>(sg, m0 + sub, r, n0, red);
  }
}

// Persistent: workgroup b takes tile b first, then pops tiles gridDim.x, gridDim.x + 1, ... from
// the list's queue counter (zeroed by the selection kernel), so a launch whose tiles all fit in
// one round makes no atomic at all.  The segments' first tiles are staged in LDS once.
template <bool GU, int MQMAX, bool W4 = false>
__global__ __launch_bounds__(256) void gemm_stream_bf16(const Seg* __restrict__ segs,
                                                         int32_t* __restrict__ meta) {
  constexpr int MQ = MQMAX > 0 ? MQMAX : 1;
  __shared__ int slot;
  __shared__ int seg_base[kSegCap];
  // split-K partials of wavefronts 1..3: up to MQ token groups x 4 x 2 floats per lane
  __shared__ float red[3 * MQ * 4 * 2 * 64];
  // MQMAX = 0: the activations of a one-row tile
  __shared__ __attribute__((aligned(16))) char xs[MQMAX == 0 ? kStreamXlMaxK * 2 : 16];
  extern __shared__ __attribute__((aligned(16))) uint8_t w4_sc[];  // mxfp4: staged scales
  const int nseg = meta[0], ntiles = meta[1];
  if ((int)blockIdx.x >= ntiles) return;
  for (int i = threadIdx.x; i < nseg; i += 256) seg_base[i] = segs[i].tile_base;
  __syncthreads();
  int t = blockIdx.x;
  for (;;) {
    const Seg& sg = segs[__builtin_amdgcn_readfirstlane(find_seg_lds(seg_base, nseg, t))];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    const int m0 = mt * kStreamMaxRows;
    const int rows = min(kStreamMaxRows, sg.rows - m0);
    const int n0 = nt * sg.tn;
    // long K: 16 columns per wavefront group, 4-way split in K; else 32 columns, wavefront pairs
    // (mxfp4 tiles are twice as wide)
    if ((W4 ? sg.tn / 2 : sg.tn) == 16)
      stream_rows_bf16<GU, 4, MQMAX, W4>(sg, m0, rows, n0, red, xs, w4_sc);
    else
      stream_rows_bf16<GU, 2, MQMAX, W4>(sg, m0, rows, n0, red, xs, w4_sc);
    t = gridDim.x + __builtin_amdgcn_readfirstlane(pop_tile(&meta[kMetaQueue], &slot));
    if (t >= ntiles) break;
  }
}

// ------------------------------------------------------------------------------------------------
// LDS-tiled MFMA family
//
// A tile is 256 weight rows (gate/up: 128 gate + 128 up rows -> 128 h columns; down: 256 y columns)
// by a tile height of token rows chosen from the rows the tile holds: 256 (full), 128, 64 or 32.  The
// last m-tile of an expert and every expert with at most 128 rows take the shortest height that
// holds their rows, so a 40-row expert runs a quarter of the MFMAs of a full tile and its weights
// stream at the rate of the loads instead of the MFMAs.
//  * full: 4 wavefronts as 2 (tokens) x 2 (weights), each 128 x 128 with MFMA 32x32x16: 16
//    accumulator blocks, 4 A and 4 B fragments per k-substep, every fragment reused 4 times; two
//    LDS stages of 64 KB.
//  * short (128, 64 or 32 rows): the 4 wavefronts split the weight rows (gate/up: 32 gate + 32 up
//    rows each, down: 64 rows each) and each covers every token row; three LDS stages of 48 or
//    40 KB, four of 36 KB for 32 rows, since these tiles wait on the weight stream rather than on
//    the MFMAs.
// Within a tile every MFMA runs whatever its rows (skipping empty 32-row token blocks inside a full
// tile was measured: ~3% on many-expert prefill, -2% on 8-expert prefill and ~40% more gate/up L2
// miss traffic).
//
// Scheduling: one persistent workgroup per CU.  Tiles are handed out in one of three orders chosen
// by the selection kernel (select_dev.h): light tiles spread between heavy ones; two classes with a
// queue each on every XCD, part of each XCD's CUs on full-height tiles and the rest on short ones
// (long K); or, for GEMMs of few rounds, longest first.  Within a segment the m-tiles of one weight
// tile are next to each other; consecutive runs of tiles go to one XCD, so tiles that share weight
// and activation tiles run side by side on the same L2.  A workgroup whose XCD's queues are empty
// takes work from the other XCDs' queues.  Tiles past the last whole round of CUs may be split in
// K (see kernels.h).
// ------------------------------------------------------------------------------------------------
constexpr int BM = kMfmaBM;
constexpr int BNW = 256;                  // weight rows per tile
constexpr int LROWS = BM + BNW;           // LDS rows per stage of a full tile

// Direct stores from the accumulators (the split-K epilogue kernel, which has no staging ring; the
// persistent MFMA kernel stages its tiles through LDS, MfmaTileStoreLds).
template <bool GU>
__device__ __forceinline__ void MfmaTileStore(const f32x16 (&acc)[4][4], void* out, int N, int row0,
                                              int m0, int rows, int n0) {
    const uint32_t tid = tid_here();
    const int lane = tid & 63, wv = tid >> 6;
    const int wm = wv & 1, wn = wv >> 1;
    const int l32 = lane & 31, khalf = lane >> 5;
    // lane holds C[8*(r/4) + 4*khalf + r%4][l32] of each 32x32 block (rows = weights)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = wm * 128 + b * 32 + l32;
      if (r >= rows) continue;
      const size_t orow = (size_t)(row0 + m0 + r) * N;  // element offset of the output row
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
            gstore8(out, (orow + c0 + q * 8) * 2, pk);
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
            gstore8(out, (orow + c0 + q * 8) * 2, pk);
          }
        }
      }
    }
  }

// Short tiles of TB * 32 token rows: wavefront wn holds weight blocks acc[0..1][*] (gate/up: its 32
// gate rows in block 0 and the matching 32 up rows in block 1 -> h columns [32 wn, +32); down: y
// columns [64 wn, +64)) for token blocks acc[*][0..TB).
template <bool GU, int TB>
__device__ __forceinline__ void MfmaTileStoreShort(const f32x16 (&acc)[4][4], void* out, int N,
                                                   int row0, int m0, int rows, int n0) {
  const uint32_t tid = tid_here();
  const int lane = tid & 63, wn = tid >> 6;
  const int l32 = lane & 31, khalf = lane >> 5;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const int r = b * 32 + l32;
    if (r >= rows) continue;
    const size_t orow = (size_t)(row0 + m0 + r) * N;
    if (GU) {
      const int c0 = n0 + wn * 32 + khalf * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) v[s] = swiglu(acc[0][b][q * 4 + s], acc[1][b][q * 4 + s]);
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        gstore8(out, (orow + c0 + q * 8) * 2, pk);
      }
    } else {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int cb = n0 + wn * 64 + a * 32;
        if (cb >= N) continue;
        const int c0 = cb + khalf * 4;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 pk;
          pk.x = pack_bf16x2(acc[a][b][q * 4 + 0], acc[a][b][q * 4 + 1]);
          pk.y = pack_bf16x2(acc[a][b][q * 4 + 2], acc[a][b][q * 4 + 3]);
          gstore8(out, (orow + c0 + q * 8) * 2, pk);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Memory pipeline: K-steps of 64 (128-byte LDS rows) through a ring of stages; each stage holds the
// tile's token rows, then its 256 weight rows.  Global data goes straight into LDS
// (global_load_lds_dwordx4, no staging registers), every instruction moving 8 whole 128-byte lines.
// Rows keep 8 chunks of 16 B XOR-swizzled by (row >> 1) & 7, so the 16 lanes a ds_read_b128 serves
// together (16 rows, one chunk index) cover all 64 banks.
//
// Full tiles: two stages of 64 KB.  Waits are explicit (vmcnt) around a plain barrier so prefetches
// stay in flight.  Step kt
// on stage S: substeps 0..2 run while substeps 1..3 are read; wait until this wavefront's reads are
// done and every load it issued has landed; barrier (stage S^1 complete, stage S free); half the
// loads for step kt+2 into stage S while substep 3 runs and substep 0 of stage S^1 is read, the
// other half during substep 1 of step kt+1.
//
// Short tiles: NS stages (three; four for 32-row tiles) at a run-time stage index, so that NS - 1
// steps of loads stay in flight while one stage is read.  Step kt reads stage kt % NS; before the
// barrier it waits until the loads of step kt+1 have landed (later ones may still fly), then loads
// step kt+NS into the stage it just finished.
// ------------------------------------------------------------------------------------------------
constexpr int BK64 = 64;
constexpr int ROWB64 = 128;
constexpr int STAGE64 = LROWS * ROWB64;            // 64 KB
constexpr int DMA64 = STAGE64 / (256 * 16);        // 16 loads per thread per stage
constexpr int kShortStages = 3;
constexpr int kRingBytes = kShortStages * (128 + BNW) * ROWB64;  // 144 KB (>= 2 full stages)
// LDS stages of a short tile of TB token blocks: as many as the ring holds (32-row tiles: four
// 36 KB stages, three K-steps of loads in flight; 64- and 128-row tiles: three).
template <int TB> constexpr int kStagesFor = kRingBytes / ((TB * 32 + BNW) * ROWB64) >= 4 ? 4 : 3;
static_assert(kStagesFor<1> * (32 + BNW) * ROWB64 <= kRingBytes, "32-row stages fit the ring");
// Tile height for a tile holding `rows` token rows (the shortest that fits).
__device__ __forceinline__ int tile_height(int rows) {
  return rows <= 32 ? 32 : rows <= 64 ? 64 : rows <= 128 ? 128 : kMfmaBM;
}
static_assert(kRingBytes >= 2 * STAGE64, "ring holds two full-tile stages");
__shared__ __attribute__((aligned(1024))) uint8_t g_ring[kRingBytes];
template <int S> __device__ __forceinline__ uint8_t* stage64_ptr() { return g_ring + S * STAGE64; }

// Epilogue through LDS.  Stored straight from the accumulators, a lane writes 8 bytes (4 columns)
// of each of 32 token rows per instruction: a full tile took 64 such stores per lane, and since
// stores and loads share one counter, the next tile's first wait waited for them all.  Instead the
// tile (bf16, after SwiGLU for gate/up) goes into the idle ring as [token row][column] with 16 bytes
// of padding per row (conflict-free 8-byte writes), and then every thread stores 16-byte chunks of
// whole rows: a wavefront writes two or four contiguous row segments of 256 or 512 bytes.  TB: token
// blocks of a short tile (8: a full tile).  The ring is idle: the K loop ended with a wait and a
// barrier, and the next tile's loads go out after the claim's barrier.

template <bool GU, int TB>
__device__ __forceinline__ void MfmaTileStoreLds(const f32x16 (&acc)[4][4], void* out, int N, int row0,
                                                 int m0, int rows, int n0) {
  constexpr bool kFull = TB == 8;
  constexpr int W = GU ? 128 : 256;  // the tile's output columns
  constexpr int RS = W * 2 + 16;     // LDS row stride in bytes
  static_assert(256 * RS <= kRingBytes, "an output tile fits the ring");
  const uint32_t tid = tid_here();
  const int lane = tid & 63, wv = tid >> 6;
  const int l32 = lane & 31, khalf = lane >> 5;
  auto put = [&](int t, int col, float v0, float v1, float v2, float v3) {
    uint2 pk;
    pk.x = pack_bf16x2(v0, v1);
    pk.y = pack_bf16x2(v2, v3);
    *reinterpret_cast<uint2*>(g_ring + t * RS + col * 2) = pk;
  };
  // lane holds C[8*(r/4) + 4*khalf + r%4][l32] of each 32x32 block (rows = weights)
  if (kFull) {
    const int wm = wv & 1, wn = wv >> 1;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int t = wm * 128 + b * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GU) {
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            float v[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) v[s] = swiglu(acc[a][b][q * 4 + s], acc[a + 2][b][q * 4 + s]);
            put(t, wn * 64 + a * 32 + 8 * q + 4 * khalf, v[0], v[1], v[2], v[3]);
          }
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a)
            put(t, wn * 128 + a * 32 + 8 * q + 4 * khalf, acc[a][b][q * 4], acc[a][b][q * 4 + 1],
                acc[a][b][q * 4 + 2], acc[a][b][q * 4 + 3]);
        }
      }
    }
  } else {
    const int wn = wv;
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int t = b * 32 + l32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GU) {
          float v[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) v[s] = swiglu(acc[0][b][q * 4 + s], acc[1][b][q * 4 + s]);
          put(t, wn * 32 + 8 * q + 4 * khalf, v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int a = 0; a < 2; ++a)
            put(t, wn * 64 + a * 32 + 8 * q + 4 * khalf, acc[a][b][q * 4], acc[a][b][q * 4 + 1],
                acc[a][b][q * 4 + 2], acc[a][b][q * 4 + 3]);
        }
      }
    }
  }
  __syncthreads();
  constexpr int CPR = W / 8;      // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;  // rows per pass of the workgroup
  constexpr int H = kFull ? 256 : TB * 32;
  const int c = tid % CPR;
  const int col = n0 + c * 8;
  const int nr = rows < H ? rows : H;
  if (col < N) {  // (down: the last tile of a row may be half full)
    for (int t = tid / CPR; t < nr; t += RPP) {
      const uint4 v = *reinterpret_cast<const uint4*>(g_ring + t * RS + c * 16);
      // h is read back by the down GEMM right away; y only by the combine, after the whole GEMM
      if (GU) gstore16(out, ((size_t)(row0 + m0 + t) * N + col) * 2, v);
      else gstore16_nt(out, ((size_t)(row0 + m0 + t) * N + col) * 2, v);
    }
  }
}

__device__ __forceinline__ int lds_off64(int r, int c) { return r * ROWB64 + ((c ^ ((r >> 1) & 7)) << 4); }

// Fragment reads: a wavefront's A (weight) and B (token) fragments sit in 32-row blocks starting at
// multiples of 32 rows, so a lane's swizzle (row >> 1) & 7 = (lane % 32 >> 1) & 7 is the same in
// every block.  Each read address is then a per-lane base for the k-substep (row 32*blk + lane%32,
// chunk 2*kk + lane/32) plus a block offset that is a compile-time constant, which the LDS read
// instruction carries as its immediate: 4 bases per operand instead of one register per fragment.
__device__ __forceinline__ int frag_lane_off(int kk) {
  const int lane = threadIdx.x & 63, l32 = lane & 31;
  return l32 * ROWB64 + (((kk * 2 + (lane >> 5)) ^ ((l32 >> 1) & 7)) << 4);
}
// byte offset of weight block a of a full tile (gate/up: gate blocks 0, 1 then up blocks 2, 3)
template <bool GU>
__device__ __forceinline__ constexpr int full_a_blk(int a) {
  return GU ? ((a & 1) * 32 + (a >> 1) * 128) * ROWB64 : a * 32 * ROWB64;
}

template <bool GU>
struct MfmaTile {
  // Load slot j of wavefront wv fills LDS rows [32*j + 8*wv, +8) of a stage: slots [0, NTS) token
  // rows, then 8 slots of weight rows (gate/up: 4 of gate rows 0..127, 4 of up rows 0..127), with
  // NTS = tile height / 32.
  const char* abase;
  const char* wbase0;
  const char* wbase1;
  uint32_t off[DMA64];
  int wvu;
  int bm;  // tile height: 256, 128, 64 or 32 token rows
  int arow0, brow0;  // LDS byte offsets of the wavefront's first weight and token rows
  f32x16 acc[4][4];

  template <int NTS>
  __device__ __forceinline__ const char* slot_base(int j) const {
    return j < NTS ? abase : ((!GU || j < NTS + 4) ? wbase0 : wbase1);
  }

  // kt0: first 64-wide K-step of the tile's K range (a piece of a split tile starts past 0)
  __device__ __forceinline__ void setup(const Seg& sg, int m0, int rows, int n0, int kt0) {
    const int lane = tid_here() & 63;  // (lane constants stay in the claim, not held across tiles)
    wvu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    bm = tile_height(rows);
    const int nts = bm >> 5;
    const uint32_t rowbytes = (uint32_t)sg.K * 2;
    abase = static_cast<const char*>(sg.a);
    wbase0 = static_cast<const char*>(sg.w0);
    wbase1 = static_cast<const char*>(GU ? sg.w1 : sg.w0);
    // Token rows of slots 0..7, fetched together whatever the tile height (slots at or past NTS
    // are weight slots and drop theirs).  Padded rows (r >= rows) all read the first row's first 16
    // bytes: one coalesced request per instruction instead of eight lines; their LDS rows are never
    // stored.
    int src[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 32 * j + 8 * wvu + (lane >> 3);
      src[j] = sg.row0 + m0 + (r < rows ? r : 0);
    }
    if (sg.tok) {
#pragma unroll
      for (int j = 0; j < 8; ++j) src[j] = gload_i32(sg.tok, src[j]);
    }
#pragma unroll
    for (int j = 0; j < DMA64; ++j) {
      const int r = 32 * j + 8 * wvu + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      // as a weight slot, LDS row r holds the tile's weight row r - bm (slots past the tile's last
      // weight slot are never issued)
      int wr = GU ? n0 + ((r - bm) & 127) : n0 + (r - bm);
      wr = wr < sg.N ? wr : sg.N - 1;
      const uint32_t woff = (uint32_t)wr * rowbytes + c * 16 + (uint32_t)kt0 * ROWB64;
      if (j < 8) {
        const int rr = 32 * j + 8 * wvu + (lane >> 3);
        const uint32_t toff =
            (uint32_t)src[j] * rowbytes + (rr < rows ? c * 16 + (uint32_t)kt0 * ROWB64 : 0);
        off[j] = j < nts ? toff : woff;
      } else {
        off[j] = woff;
      }
    }
    if (bm == BM) {
      const int wm = wvu & 1, wn = wvu >> 1;
      arow0 = (BM + (GU ? wn * 64 : wn * 128)) * ROWB64;
      brow0 = wm * 128 * ROWB64;
    } else {
      const int wn = wvu;
      arow0 = (bm + (GU ? wn * 32 : wn * 64)) * ROWB64;
      brow0 = 0;
    }
  }

  // ---- full tiles ----
  template <int S>
  __device__ __forceinline__ void issue_one(int j, uint32_t ko) {
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t* st = stage64_ptr<S>() + wv * 8 * ROWB64;
    dma16(slot_base<8>(j) + ko, off[j], (lds_void*)(st + j * 32 * ROWB64));
  }

  template <int S>
  __device__ __forceinline__ void issue(int kt) {
#pragma unroll
    for (int j = 0; j < DMA64; ++j) issue_one<S>(j, (uint32_t)kt * ROWB64);
  }

  // fragment i of a full tile's k-substep (0..3: weight blocks, 4..7: token blocks)
  __device__ __forceinline__ bf16x8 frag_full(const uint8_t* st, int va, int vb, int i) const {
    const uint8_t* p = i < 4 ? st + va + full_a_blk<GU>(i) : st + vb + (i - 4) * 32 * ROWB64;
    return as_bf16x8(*reinterpret_cast<const uint4*>(p));
  }

  template <int S>
  __device__ __forceinline__ void read_frags(int kk, bf16x8 (&f)[8]) const {
    const uint8_t* st = stage64_ptr<S>();
    const int lo = frag_lane_off(kk), va = arow0 + lo, vb = brow0 + lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = frag_full(st, va, vb, i);
  }

  __device__ __forceinline__ void mfmas(const bf16x8 (&f)[8]) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(f[a], f[4 + b], acc[a][b]);
  }

  // 16 MFMAs with the 8 fragment reads issued behind the first 8
  template <int S>
  __device__ __forceinline__ void sub(int kk, const bf16x8 (&cur)[8], bf16x8 (&nxt)[8]) {
    __builtin_amdgcn_sched_barrier(0);
    read_frags<S>(kk, nxt);
    mfmas(cur);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // The same with loads J0 .. J0 + N - 1 of the K-step at offset ko (into stage T), one per MFMA:
  // gate/up places them on the first N MFMAs, beside the fragment reads, down on the last N, the
  // faster placement for each (the scheduler cannot see the asm loads, so the interleave is fixed
  // by hand).
  template <int S, int T, int J0, int N>
  __device__ __forceinline__ void sub_dma(int kk, const bf16x8 (&cur)[8], bf16x8 (&nxt)[8], uint32_t ko) {
    const uint8_t* st = stage64_ptr<S>();
    const int lo = frag_lane_off(kk), va = arow0 + lo, vb = brow0 + lo;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      constexpr int L0 = GU ? 0 : 16 - N;  // first MFMA with a load
      if (i >= L0 && i < L0 + N) issue_one<T>(J0 + i - L0, ko);
      if (i < 8) nxt[i] = frag_full(st, va, vb, i);
      acc[i >> 2][i & 3] = mfma32(cur[i >> 2], cur[4 + (i & 3)], acc[i >> 2][i & 3]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // The 16 loads of a K-step go out in two halves: kDma0 behind the MFMAs of the previous step's
  // substep 3 (right after its barrier), the rest behind substep 1 of the step before the one
  // that reads them.  Issued all at once after the barrier, the four wavefronts' 64 loads queued
  // behind each other and held up the MFMAs interleaved with them (Mixtral-shaped layer 2.68 ->
  // 2.58 ms); issuing any of them later than substep 1 left too little time for them to land.
  // (At a tile's first step the second half repeats loads of the prologue.)
  static constexpr int kDma0 = 8;

  template <int S>
  __device__ __forceinline__ void step(int kt, int nk, bf16x8 (&f0)[8], bf16x8 (&f1)[8]) {
    // the rest of step kt+1's loads (into stage S^1)
    const uint32_t k1 = (uint32_t)min(kt + 1, nk - 1) * ROWB64;
    sub_dma<S, S ^ 1, kDma0, DMA64 - kDma0>(1, f0, f1, k1);
    sub<S>(2, f1, f0);
    sub<S>(3, f0, f1);
    MOE_WAITCNT(0, 0);
    __builtin_amdgcn_s_barrier();
    // the first kDma0 loads for step kt+2, with substep 0 of stage S^1 read behind the first eight
    // MFMAs of substep 3
    const uint32_t ko = (uint32_t)min(kt + 2, nk - 1) * ROWB64;
    const uint8_t* rd = stage64_ptr<S ^ 1>();
    const int lo = frag_lane_off(0), va = arow0 + lo, vb = brow0 + lo;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i < kDma0) issue_one<S>(i, ko);
      acc[i >> 2][i & 3] = mfma32(f1[i >> 2], f1[4 + (i & 3)], acc[i >> 2][i & 3]);
      if (i < 8) f0[i] = frag_full(rd, va, vb, i);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ void prologue_full() {
    issue<0>(0);
    issue<1>(1);
  }

  // nk: K-steps of the tile's K range (even)
  __device__ __forceinline__ void run_full(int nk) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    MOE_WAITCNT(DMA64, 15);  // stage 0 (the oldest loads) has landed
    __builtin_amdgcn_s_barrier();
    bf16x8 f0[8], f1[8];
    read_frags<0>(0, f0);
    for (int kt = 0; kt < nk; kt += 2) {
      step<0>(kt, nk, f0, f1);
      step<1>(kt + 1, nk, f0, f1);
    }
    MOE_WAITCNT(0, 0);
    __builtin_amdgcn_s_barrier();
  }

  // ---- short tiles (TB = tile height / 32 token blocks) ----
  template <int TB>
  __device__ __forceinline__ void issue_short_one(int stage, int j, uint32_t ko) {
    constexpr int kStage = (TB * 32 + BNW) * ROWB64;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t* st = g_ring + stage * kStage + wv * 8 * ROWB64;
    // The gate/up weights of a short tile stream with the non-temporal policy: a light expert's
    // weight rows are read by this tile alone, and left in L2 they only push out the tiles that
    // full-height neighbours share (DeepSeek-V3-shaped decode at T = 64 and 256: gate/up -9%).
    // Not the down weights: there the mixed order keeps an expert's short last m-tile next to
    // its full-height siblings, which read the same weight rows (Kimi-K2-shaped down GEMM +7%).
    if (GU && j >= TB) dma16<true>(slot_base<TB>(j) + ko, off[j], (lds_void*)(st + j * 32 * ROWB64));
    else dma16(slot_base<TB>(j) + ko, off[j], (lds_void*)(st + j * 32 * ROWB64));
  }

  template <int TB>
  __device__ __forceinline__ void issue_short(int stage, int kt) {
#pragma unroll
    for (int j = 0; j < TB + 8; ++j) issue_short_one<TB>(stage, j, (uint32_t)kt * ROWB64);
  }

  // fragment i of a short tile's k-substep (0, 1: weight blocks -- gate/up: 32 gate rows, then the
  // matching up rows 128 further; down: two consecutive blocks -- 2..: token blocks)
  template <int TB>
  __device__ __forceinline__ bf16x8 frag_short(const uint8_t* st, int va, int vb, int i) const {
    const uint8_t* p = i < 2 ? st + va + i * (GU ? 128 : 32) * ROWB64 : st + vb + (i - 2) * 32 * ROWB64;
    return as_bf16x8(*reinterpret_cast<const uint4*>(p));
  }

  template <int TB>
  __device__ __forceinline__ void read_frags_short(const uint8_t* st, int kk, bf16x8 (&f)[2 + TB]) const {
    const int lo = frag_lane_off(kk), va = arow0 + lo, vb = brow0 + lo;
#pragma unroll
    for (int i = 0; i < 2 + TB; ++i) f[i] = frag_short<TB>(st, va, vb, i);
  }

  template <int TB>
  __device__ __forceinline__ void mfmas_short(const bf16x8 (&f)[2 + TB]) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < TB; ++b) acc[a][b] = mfma32(f[a], f[2 + b], acc[a][b]);
  }

  template <int TB>
  __device__ __forceinline__ void sub_short(const uint8_t* st, int kk, const bf16x8 (&cur)[2 + TB],
                                            bf16x8 (&nxt)[2 + TB]) {
    __builtin_amdgcn_sched_barrier(0);
    read_frags_short<TB>(st, kk, nxt);
    mfmas_short<TB>(cur);
    constexpr int kPairs = 2 * TB < 2 + TB ? 2 * TB : 2 + TB;
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (2 * TB > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, 2 * TB - kPairs, 0);
    if constexpr (2 + TB > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, 2 + TB - kPairs, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int TB>
  __device__ __forceinline__ void prologue_short(int nk) {
#pragma unroll
    for (int s = 0; s < kStagesFor<TB>; ++s) issue_short<TB>(s, min(s, nk - 1));
  }

  template <int TB>
  __device__ __forceinline__ void run_short(int nk) {
    constexpr int kStage = (TB * 32 + BNW) * ROWB64;
    constexpr int D = TB + 8;  // loads per thread per stage
    constexpr int NS = kStagesFor<TB>;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    MOE_WAITCNT((NS - 1) * D, 15);  // stage 0 (the oldest loads) has landed
    __builtin_amdgcn_s_barrier();
    bf16x8 f0[2 + TB], f1[2 + TB];
    read_frags_short<TB>(g_ring, 0, f0);
    int s = 0;
    for (int kt = 0; kt < nk; ++kt) {
      const uint8_t* st = g_ring + s * kStage;
      sub_short<TB>(st, 1, f0, f1);
      sub_short<TB>(st, 2, f1, f0);
      sub_short<TB>(st, 3, f0, f1);
      // this wavefront's reads of stage s are done and its loads for step kt+1 have landed
      MOE_WAITCNT((NS - 2) * D, 0);
      __builtin_amdgcn_s_barrier();
      // the loads for step kt+NS into stage s, interleaved with the MFMAs of substep 3 and the
      // reads of substep 0 of the next stage
      const uint32_t ko = (uint32_t)min(kt + NS, nk - 1) * ROWB64;
      const int sn = s == NS - 1 ? 0 : s + 1;
      const uint8_t* rd = g_ring + sn * kStage;
      const int lo = frag_lane_off(0), va = arow0 + lo, vb = brow0 + lo;
#pragma unroll
      for (int i = 0; i < D; ++i) {
        __builtin_amdgcn_sched_barrier(0);
        issue_short_one<TB>(s, i, ko);
        if (i < 2 * TB) acc[i / TB][i % TB] = mfma32(f1[i / TB], f1[2 + i % TB], acc[i / TB][i % TB]);
        if (i < 2 + TB) f0[i] = frag_short<TB>(rd, va, vb, i);
      }
      __builtin_amdgcn_sched_barrier(0);
      s = sn;
    }
    MOE_WAITCNT(0, 0);
    __builtin_amdgcn_s_barrier();
  }

  __device__ __forceinline__ void prologue(int nk) {
    if (bm == BM) prologue_full();
    else if (bm == 128) prologue_short<4>(nk);
    else if (bm == 64) prologue_short<2>(nk);
    else prologue_short<1>(nk);
  }
};

// A piece of a split tile (accumulator blocks a < NA, b < NB) writes its partial sums to its slot of
// the tile's S slots; mfma_split_epilogue adds them later.  Slot layout: 4 accumulators (16 B) per
// thread, threads adjacent, so each store is one contiguous kilobyte per wavefront; group (a, b, q)
// of a slot starts at float (a*16+b*4+q)*1024.  Group bases are uniform; the lane's offset is one
// register, produced by asm so that the compiler cannot fold it into 64 per-group addresses hoisted
// out of the tile loop (they would not fit in registers).
template <int NA, int NB>
__device__ __forceinline__ void split_store(const f32x16 (&acc)[4][4], float* tile_part, int piece) {
  uint32_t lane_off;
  asm volatile("v_lshlrev_b32 %0, 4, %1" : "=v"(lane_off) : "v"((uint32_t)threadIdx.x));
  float* mine = tile_part + (size_t)piece * kSplitSlotFloats;
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint4 v;
        v.x = __float_as_uint(acc[a][b][q * 4 + 0]);
        v.y = __float_as_uint(acc[a][b][q * 4 + 1]);
        v.z = __float_as_uint(acc[a][b][q * 4 + 2]);
        v.w = __float_as_uint(acc[a][b][q * 4 + 3]);
        gstore16(mine + ((a * 4 + b) * 4 + q) * 1024, lane_off, v);
      }
}

// The claimed tile.  The epilogue's fields are copied here so that it reads no Seg memory after
// the next tile's loads were issued (a vector load would wait for them).  piece: -1 for a whole
// tile, else the piece of split tile u, covering K-steps [piece * nk, (piece + 1) * nk).
struct MfmaCur { int m0, rows, n0, h, nk, N, row0, piece, u; void* out; };

// One MFMA list's queue as the persistent loop sees it (positions: [0, sbase) whole tiles, then S
// pieces for each tile of [sbase, ntiles)).
struct MfmaQueue {
  const Seg* segs;
  int32_t* queues;
  int32_t* queues1;     // class-1 queues of the two-class order
  const int* seg_base;  // LDS: first tile of each segment
  int nseg, ntiles, ntiles0, sbase, S, nq, chunk;
  int order;  // TileOrder
  int pref, b0, b1;  // two-class order: this workgroup's first class, the classes' XCD chunks
};

// The persistent tile loop.  Instantiated with and without the split-K epilogue, so that lists that
// split nothing (the common case) run code whose registers the split path does not disturb.
template <bool GU, bool kSplit>
__device__ __forceinline__ void mfma_persistent(const MfmaQueue& Q, float* split_part, int* slot) {
  int q = 0;
  MfmaTile<GU> tile;
  auto claim = [&](MfmaCur& c) -> bool {
    // (the queue's counts go through opaque moves: the reciprocals of its integer divisions are
    // then computed here per claim instead of being hoisted and held across the K loops)
    const int ntiles = opaque_s(Q.ntiles), ntiles0 = opaque_s(Q.ntiles0), chunk = opaque_s(Q.chunk);
    c.piece = -1;
    c.u = 0;
    int t;
    if (!kSplit && Q.order == kOrderTwoClass) {  // (lists of that order split nothing)
      t = pop_tile_two_class(Q.queues, Q.queues1, ntiles0, ntiles - ntiles0, opaque_s(Q.b0),
                             opaque_s(Q.b1), Q.pref, slot, q);
      if (t < 0) return false;
    } else {
      const int pos = pop_tile_xcd(Q.queues, kSplit ? opaque_s(Q.nq) : ntiles, chunk, slot, q);
      if (pos < 0) return false;
      int tp = pos;
      if (kSplit && pos >= Q.sbase) {
        const int S = opaque_s(Q.S);
        c.u = (pos - Q.sbase) / S;
        c.piece = pos - Q.sbase - c.u * S;
        tp = Q.sbase + c.u;
      }
      // (a split list of the two-class order, which has less than one round, takes the mixed one)
      t = Q.order == kOrderLongestFirst ? tp : interleave_tile(tp, ntiles0, ntiles);
    }
    const int si = __builtin_amdgcn_readfirstlane(find_seg_lds(Q.seg_base, Q.nseg, t));
    const Seg& sg = Q.segs[si];
    const int local = t - sg.tile_base;
    const int mt = local % sg.mtiles, nt = local / sg.mtiles;
    c.m0 = mt * BM;
    c.rows = min(BM, sg.rows - c.m0);
    c.n0 = nt * (GU ? kMfmaBNGateUp : kMfmaBNDown);
    const int nkt = sg.K / BK64;
    c.nk = c.piece < 0 ? nkt : nkt / Q.S;
    c.N = sg.N;
    c.row0 = sg.row0;
    c.out = sg.out;
    tile.setup(sg, c.m0, c.rows, c.n0, c.piece < 0 ? 0 : c.piece * c.nk);
    c.h = __builtin_amdgcn_readfirstlane(tile.bm);
    tile.prologue(c.nk);
    return true;
  };
  auto part = [&](const MfmaCur& c) { return split_part + (size_t)c.u * Q.S * kSplitSlotFloats; };
  MfmaCur cur;
  if (!claim(cur)) return;
  for (;;) {
    // run, then this tile's epilogue, then the next claim; each height has its own branch so the
    // accumulators a shorter tile leaves unused are dead around the loop.  (Claiming the next tile
    // before the epilogue, so that its prologue loads fly during the stores, measured 1% slower
    // on the Mixtral- and Kimi-shaped prefill layers.)
    if (cur.h == BM) {
      tile.run_full(cur.nk);
      if (!kSplit || cur.piece < 0)
        MfmaTileStoreLds<GU, 8>(tile.acc, cur.out, cur.N, cur.row0, cur.m0, cur.rows, cur.n0);
      else
        split_store<4, 4>(tile.acc, part(cur), cur.piece);
    } else if (cur.h == 128) {
      tile.template run_short<4>(cur.nk);
      if (!kSplit || cur.piece < 0)
        MfmaTileStoreLds<GU, 4>(tile.acc, cur.out, cur.N, cur.row0, cur.m0, cur.rows, cur.n0);
      else
        split_store<2, 4>(tile.acc, part(cur), cur.piece);
    } else if (cur.h == 64) {
      tile.template run_short<2>(cur.nk);
      if (!kSplit || cur.piece < 0)
        MfmaTileStoreLds<GU, 2>(tile.acc, cur.out, cur.N, cur.row0, cur.m0, cur.rows, cur.n0);
      else
        split_store<2, 2>(tile.acc, part(cur), cur.piece);
    } else {
      tile.template run_short<1>(cur.nk);
      if (!kSplit || cur.piece < 0)
        MfmaTileStoreLds<GU, 1>(tile.acc, cur.out, cur.N, cur.row0, cur.m0, cur.rows, cur.n0);
      else
        split_store<2, 1>(tile.acc, part(cur), cur.piece);
    }
    if (!claim(cur)) break;
  }
}

template <bool GU>
__global__ __launch_bounds__(256, 1) void gemm_mfma_bf16(const Seg* __restrict__ segs,
                                                          int32_t* __restrict__ meta,
                                                          float* __restrict__ split_part) {
  __shared__ int slot;
  __shared__ int seg_base[kSegCap];
  MfmaQueue Q;
  Q.ntiles = meta[1];
  if (Q.ntiles == 0) return;
  Q.segs = segs;
  Q.queues = meta + kMetaQueue;
  Q.queues1 = meta + kMetaQueue1;
  Q.seg_base = seg_base;
  Q.nseg = meta[0];
  Q.ntiles0 = meta[kMetaClass0];
  Q.order = meta[kMetaOrder];
  {
    // two-class order: the first r0 workgroups of each XCD start on class 0, in proportion to the
    // classes' estimated CU time; each class's XCD chunk is the number of CUs that start on it
    const int g = max(1, (int)gridDim.x / kXcds), n0 = Q.ntiles0, n1 = Q.ntiles - Q.ntiles0;
    const long long w0 = (long long)kTwoClassW0 * n0, w1 = (long long)kTwoClassW1 * n1;
    int r0 = n1 == 0 ? g : n0 == 0 ? 0 : (int)((g * w0 + (w0 + w1) / 2) / (w0 + w1));
    if (n0 > 0 && n1 > 0) r0 = min(max(r0, 1), g - 1);
    Q.pref = (int)(blockIdx.x / kXcds) < r0 ? 0 : 1;
    Q.b0 = max(r0, 1);
    Q.b1 = max(g - r0, 1);
  }
  Q.sbase = meta[kMetaSplitBase];
  Q.S = meta[kMetaSplitS];
  Q.nq = Q.sbase + (Q.ntiles - Q.sbase) * Q.S;
  // XCD chunk of the one-queue orders: twice the CUs of an XCD for the mixed order (DeepSeek-V3-
  // shaped decode at T = 256: down GEMM 2.5-4.6% faster, other shapes unchanged), one round of
  // them otherwise
  Q.chunk = __builtin_amdgcn_readfirstlane(max(1, (int)gridDim.x / kXcds) *
                                           (Q.order == kOrderMix ? 2 : 1));
  for (int i = threadIdx.x; i < Q.nseg; i += blockDim.x) seg_base[i] = segs[i].tile_base;
  __syncthreads();
  if (Q.S > 1) mfma_persistent<GU, true>(Q, split_part, &slot);
  else mfma_persistent<GU, false>(Q, split_part, &slot);
}

// Epilogue of the tiles split in K: workgroup u adds the S partial-sum slots of split tile u (queue
// position sbase + u) in piece order -- so the result does not depend on which piece finished
// first -- and stores the tile as the MFMA kernel would have.  It runs after the GEMM's MFMA kernel
// on the same stream; with no split tiles every workgroup returns at once.
template <bool GU>
__global__ __launch_bounds__(256, 1) void mfma_split_epilogue(const Seg* __restrict__ segs,
                                                               const int32_t* __restrict__ meta,
                                                               const float* __restrict__ split_part) {
  const int ntiles = meta[1], sbase = meta[kMetaSplitBase], S = meta[kMetaSplitS];
  const int u = blockIdx.x;
  if (S <= 1 || sbase + u >= ntiles) return;
  const int tp = sbase + u, order = meta[kMetaOrder], ntiles0 = meta[kMetaClass0];
  const int t = order == kOrderLongestFirst ? tp : interleave_tile(tp, ntiles0, ntiles);
  int lo = 0, hi = meta[0] - 1;  // the last segment whose first tile is <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].tile_base <= t) lo = mid;
    else hi = mid - 1;
  }
  const Seg& sg = segs[lo];
  const int local = t - sg.tile_base;
  const int mt = local % sg.mtiles, nt = local / sg.mtiles;
  const int m0 = mt * BM, rows = min(BM, sg.rows - m0);
  const int n0 = nt * (GU ? kMfmaBNGateUp : kMfmaBNDown);
  const int h = tile_height(rows);
  const int NA = h == BM ? 4 : 2, NB = h == BM ? 4 : h / 32;
  const float* part = split_part + (size_t)u * S * kSplitSlotFloats;
  const uint32_t lane_off = threadIdx.x * 16;
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float t4[4] = {0.f, 0.f, 0.f, 0.f};
        if (a < NA && b < NB) {
          // all pieces' loads first (S <= kSplitMaxS), then the sum in piece order
          const float* gb = part + ((a * 4 + b) * 4 + q) * 1024;
          uint4 w[kSplitMaxS];
#pragma unroll
          for (int p = 0; p < kSplitMaxS; ++p)
            if (p < S) w[p] = gload16(gb + (size_t)p * kSplitSlotFloats, lane_off);
#pragma unroll
          for (int p = 0; p < kSplitMaxS; ++p) {
            if (p >= S) break;
            const float v[4] = {__uint_as_float(w[p].x), __uint_as_float(w[p].y),
                                __uint_as_float(w[p].z), __uint_as_float(w[p].w)};
#pragma unroll
            for (int i = 0; i < 4; ++i) t4[i] = p == 0 ? v[i] : t4[i] + v[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][b][q * 4 + i] = t4[i];
      }
    }
  if (h == BM) MfmaTileStore<GU>(acc, sg.out, sg.N, sg.row0, m0, rows, n0);
  else if (h == 128) MfmaTileStoreShort<GU, 4>(acc, sg.out, sg.N, sg.row0, m0, rows, n0);
  else if (h == 64) MfmaTileStoreShort<GU, 2>(acc, sg.out, sg.N, sg.row0, m0, rows, n0);
  else MfmaTileStoreShort<GU, 1>(acc, sg.out, sg.N, sg.row0, m0, rows, n0);
}

// ------------------------------------------------------------------------------------------------
// single-token decode: routing fused into the gate/up kernel
//
// With one token, each expert's segment is one row and the rows follow the selected experts in
// increasing id (the stable permutation of the token's k slots), so a workgroup that has routed
// the token itself knows every tile's expert and row: tile t = (row t / P, columns (t % P) * tn),
// P = f / tn.  Routing is a single wavefront's work (route_dev.h) and costs each workgroup less
// than a separate front-end launch and its selection pass would cost the whole layer.
// ------------------------------------------------------------------------------------------------
template <int VPL, int WK>
__global__ __launch_bounds__(256) void decode1_gate_up_bf16(Decode1Args a, SelectOut o) {
  constexpr int tn = WK == 4 ? 16 : 32;
  __shared__ int s_ids[kMaxTopK];   // the routing, in slot order
  __shared__ int s_exp[kMaxTopK];   // the selected experts in increasing id (row order)
  __shared__ float red[3 * 4 * 2 * 64];
  __shared__ __attribute__((aligned(16))) char xs[kStreamXlMaxK * 2];
  const int tid = threadIdx.x, k = a.k;
  const int per_exp = a.f / tn, ntiles = k * per_exp;
  const bool lead = blockIdx.x == 0;
  if ((int)blockIdx.x >= ntiles) return;
  if (tid < 64) {
    route_token<VPL>(a.logits, 0, a.E, k, lead ? a.ids : nullptr, lead ? a.w : nullptr, s_ids);
  } else {  // meanwhile the other wavefronts stage the token's activations for every tile
    const uint4* xg = static_cast<const uint4*>(a.x);
    uint4* xw = reinterpret_cast<uint4*>(xs);
    for (int i = tid - 64; i < a.d / 8; i += 192) xw[i] = xg[i];
  }
  __syncthreads();
  if (tid < k) {  // the k ids are distinct: row = number of selected ids below this one
    const int e = s_ids[tid];
    int r = 0;
    for (int j = 0; j < k; ++j) r += s_ids[j] < e ? 1 : 0;
    s_exp[r] = e;
    if (lead) {
      a.perm_src[r] = tid;
      a.slot_dst[tid] = r;
      a.tok[r] = 0;
    }
  }
  if (lead) {
    for (int e = tid; e <= a.E; e += 256) {
      int below = 0, hit = 0;
      for (int j = 0; j < k; ++j) {
        below += s_ids[j] < e ? 1 : 0;
        hit |= s_ids[j] == e ? 1 : 0;
      }
      if (e < a.E) a.counts[e] = hit;
      a.offsets[e] = below;
    }
  }
  __syncthreads();
  if (lead && tid < k) {
    // the down GEMM's streaming list, as the selection writes it: one segment per row, by id
    const int r = tid, e = s_exp[r];
    const int dtn = stream_bn(a.f), dt = (a.d + dtn - 1) / dtn;
    Seg sg;
    sg.a = a.h;
    sg.tok = nullptr;
    sg.as = nullptr;
    sg.w0 = static_cast<const uint8_t*>(a.w_down) + (size_t)e * a.d * a.f * 2;
    sg.w1 = nullptr;
    sg.s0 = nullptr;
    sg.s1 = nullptr;
    sg.e0 = sg.e1 = nullptr;
    sg.ae = nullptr;
    sg.oute = nullptr;
    sg.out = a.y;
    sg.outs = nullptr;
    sg.row0 = r;
    sg.rows = 1;
    sg.N = a.d;
    sg.K = a.f;
    sg.tile_base = r * dt;
    sg.mtiles = 1;
    sg.ntiles = dt;
    sg.expert = e;
    sg.tn = dtn;
    o.segs[(size_t)(kGemmDown * kNumFam + kFamStream) * kSegCap + r] = sg;
    if (r == 0) {  // stream list: k segments, k * dt tiles, zeroed queue; MFMA list: empty
      for (int fam = 0; fam < kNumFam; ++fam) {
        int32_t* m = o.meta + (kGemmDown * kNumFam + fam) * kMetaStride;
        const bool st = fam == kFamStream;
        for (int q = 0; q < kMetaStride; ++q) m[q] = 0;
        m[0] = st ? k : 0;
        m[1] = st ? k * dt : 0;
        m[kMetaSplitS] = 1;
      }
    }
  }
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int r = t / per_exp, e = s_exp[r];
    Seg sg;
    sg.a = a.x;
    sg.tok = nullptr;
    sg.as = nullptr;
    sg.w0 = static_cast<const uint8_t*>(a.w_gate) + (size_t)e * a.f * a.d * 2;
    sg.w1 = static_cast<const uint8_t*>(a.w_up) + (size_t)e * a.f * a.d * 2;
    sg.s0 = nullptr;
    sg.s1 = nullptr;
    sg.e0 = sg.e1 = nullptr;
    sg.ae = nullptr;
    sg.oute = nullptr;
    sg.out = a.h;
    sg.outs = nullptr;
    sg.row0 = r;
    sg.rows = 1;
    sg.N = a.f;
    sg.K = a.d;
    sg.tile_base = r * per_exp;
    sg.mtiles = 1;
    sg.ntiles = per_exp;
    sg.expert = e;
    sg.tn = tn;
    stream_tile_bf16<1, true, WK, 2>(sg, 0, 1, (t - r * per_exp) * tn, red, xs);
  }
}

// ------------------------------------------------------------------------------------------------
// The whole single-token layer in one launch (MOE_CONFIG_FUSED): Weave (Abstract) runs an MoE layer
// as one persistent megakernel whose workers are scheduled over its phases, and GC-MoE (summary)
// launches its decode path as one graph.  Here every workgroup routes the token itself (as the
// single-token gate/up kernel does), takes its gate/up tiles, then its down tiles, each waiting for
// the gate/up tiles of its row through a device counter; the last down tile of each column block
// (a counter again) does the combine of that block.  Cooperative launch: every workgroup is
// resident, so the static tile assignment cannot wait on a workgroup that has not started.  Data
// that crosses XCDs (h, y) goes through device-coherent stores and loads (common.h), with the
// writer's stores drained before its counter increment; no fence writes back or invalidates an L2.
// The counters live in the first kFusedSyncInts ints of the workspace (zero before the first
// launch); each launch returns them to zero: the last down tile of a row past its wait clears that
// row's counters, the combining tile its column block's.  (A variant that handed the tiles out
// from a device ticket queue under a plain launch did not finish its first test on the GPU; its
// cause was not found, so it was dropped.)
// Counter layout (ints): the polled per-row counters 4 KB apart (so that a thousand workgroups
// polling them do not all load one memory channel), gate/up tiles finished of row r at
// kFusedSyncRow r and its down tiles past their wait 32 ints further; the error flag at
// kFusedSyncErr; down tiles finished of column block b at kFusedSyncDn + b.
constexpr int kFusedSyncRow = 1024;
constexpr int kFusedSyncErr = kMaxTopK * kFusedSyncRow;
constexpr int kFusedSyncDn = kFusedSyncErr + 32;
constexpr int kFusedMaxSpins = 1 << 20;  // ~1 s of polls: then the flag is set and the wait ends
static_assert(kFusedSyncDn + kStreamXlMaxK / 16 <= kFusedSyncInts, "fused counters");

template <int VPL, int WKG, int WKD>
__global__ __launch_bounds__(256) void decode1_fused_bf16(Decode1Args a) {
  constexpr int tn = WKG == 4 ? 16 : 32;   // gate/up tile columns
  constexpr int dtn = WKD == 4 ? 16 : 32;  // down tile columns
  __shared__ int s_ids[kMaxTopK];   // the routing, in slot order
  __shared__ float s_w[kMaxTopK];
  __shared__ int s_exp[kMaxTopK];   // the selected experts in increasing id (row order)
  __shared__ int s_row[kMaxTopK];   // slot -> row
  __shared__ int s_flag;
  __shared__ float red[3 * 4 * 2 * 64];
  __shared__ __attribute__((aligned(16))) char xs[kStreamXlMaxK * 2];
  const int tid = threadIdx.x, k = a.k;
  const int per_exp = a.f / tn, ntiles = k * per_exp;
  const int dt = a.d / dtn, ndown = k * dt;
  const bool lead = blockIdx.x == 0;
  int32_t* sync = a.sync;
  if (tid < 64) {
    route_token<VPL>(a.logits, 0, a.E, k, nullptr, s_w, s_ids);
  } else {  // meanwhile the other wavefronts stage the token's activations
    const uint4* xg = static_cast<const uint4*>(a.x);
    uint4* xw = reinterpret_cast<uint4*>(xs);
    for (int i = tid - 64; i < a.d / 8; i += 192) xw[i] = xg[i];
  }
  __syncthreads();
  if (tid < k) {  // the k ids are distinct: row = number of selected ids below this one
    const int e = s_ids[tid];
    int r = 0;
    for (int j = 0; j < k; ++j) r += s_ids[j] < e ? 1 : 0;
    s_exp[r] = e;
    s_row[tid] = r;
    if (lead) {
      a.ids[tid] = e;
      a.w[tid] = s_w[tid];
      a.perm_src[r] = tid;
      a.slot_dst[tid] = r;
      a.tok[r] = 0;
    }
  }
  if (lead) {
    for (int e = tid; e <= a.E; e += 256) {
      int below = 0, hit = 0;
      for (int j = 0; j < k; ++j) {
        below += s_ids[j] < e ? 1 : 0;
        hit |= s_ids[j] == e ? 1 : 0;
      }
      if (e < a.E) a.counts[e] = hit;
      a.offsets[e] = below;
    }
  }
  __syncthreads();
  // gate/up tiles
  for (int t = blockIdx.x; t < ntiles; t += gridDim.x) {
    // gate/up tile: h through coherent stores, then the row's counter
    const int r = t / per_exp, e = s_exp[r];
    Seg sg;
    sg.a = a.x;
    sg.tok = nullptr;
    sg.as = nullptr;
    sg.w0 = static_cast<const uint8_t*>(a.w_gate) + (size_t)e * a.f * a.d * 2;
    sg.w1 = static_cast<const uint8_t*>(a.w_up) + (size_t)e * a.f * a.d * 2;
    sg.s0 = sg.s1 = nullptr;
    sg.e0 = sg.e1 = nullptr;
    sg.ae = nullptr;
    sg.oute = nullptr;
    sg.out = a.h;
    sg.outs = nullptr;
    sg.row0 = r;
    sg.rows = 1;
    sg.N = a.f;
    sg.K = a.d;
    sg.tile_base = r * per_exp;
    sg.mtiles = 1;
    sg.ntiles = per_exp;
    sg.expert = e;
    sg.tn = tn;
    stream_tile_bf16<1, true, WKG, 2, true>(sg, 0, 1, (t - r * per_exp) * tn, red, xs);
    MOE_WAITCNT(0, 0);  // this wavefront's h stores are acknowledged
    __syncthreads();
    if (tid == 0) counter_add(&sync[kFusedSyncRow * r], 1);
  }
  __syncthreads();  // (every wavefront is done reading x from xs)
  // down tiles
  for (int t = blockIdx.x; t < ndown; t += gridDim.x) {
    // down tile: wait for the row's gate/up tiles, stage its h row, stream, count, maybe combine
    const int r = t / dt, cb = t - r * dt, e = s_exp[r];
    if (tid == 0) {
      int spins = 0;
      while (counter_load(&sync[kFusedSyncRow * r]) < per_exp) {
        if (++spins > kFusedMaxSpins) {
          counter_store(&sync[kFusedSyncErr], 1);
          break;
        }
        __builtin_amdgcn_s_sleep(32);  // (about 1 us between polls)
      }
      if (counter_add(&sync[kFusedSyncRow * r + 32], 1) == dt - 1) {  // the last waiter clears both
        counter_store(&sync[kFusedSyncRow * r], 0);
        counter_store(&sync[kFusedSyncRow * r + 32], 0);
      }
    }
    __syncthreads();
    for (int i = tid; i < a.f / 4; i += 256)
      reinterpret_cast<uint2*>(xs)[i] = gload8_coh(a.h, ((size_t)r * a.f + 4 * i) * 2);
    __syncthreads();
    Seg sg;
    sg.a = a.h;
    sg.tok = nullptr;
    sg.as = nullptr;
    sg.w0 = static_cast<const uint8_t*>(a.w_down) + (size_t)e * a.d * a.f * 2;
    sg.w1 = nullptr;
    sg.s0 = sg.s1 = nullptr;
    sg.e0 = sg.e1 = nullptr;
    sg.ae = nullptr;
    sg.oute = nullptr;
    sg.out = a.y;
    sg.outs = nullptr;
    sg.row0 = r;
    sg.rows = 1;
    sg.N = a.d;
    sg.K = a.f;
    sg.tile_base = r * dt;
    sg.mtiles = 1;
    sg.ntiles = dt;
    sg.expert = e;
    sg.tn = dtn;
    stream_tile_bf16<1, false, WKD, 2, true>(sg, 0, 1, cb * dtn, red, xs);
    MOE_WAITCNT(0, 0);  // this wavefront's y stores are acknowledged
    __syncthreads();
    if (tid == 0) s_flag = counter_add(&sync[kFusedSyncDn + cb], 1) == k - 1;
    __syncthreads();
    if (s_flag) {
      // the combine of columns [cb * dtn, +dtn), as combine_kernel: fp32 in slot order, one RNE
      if (tid < dtn / 4) {
        const int c = cb * dtn + 4 * tid;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
          const uint2 v = gload8_coh(a.y, ((size_t)s_row[j] * a.d + c) * 2);
          const float wj = s_w[j];
          acc[0] += wj * bf16_to_f32(uint16_t(v.x & 0xFFFF));
          acc[1] += wj * bf16_to_f32(uint16_t(v.x >> 16));
          acc[2] += wj * bf16_to_f32(uint16_t(v.y & 0xFFFF));
          acc[3] += wj * bf16_to_f32(uint16_t(v.y >> 16));
        }
        uint2 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        gstore8(a.out, (size_t)c * 2, o);
      }
      if (tid == 0) counter_store(&sync[kFusedSyncDn + cb], 0);
    }
    __syncthreads();  // (s_flag and xs are reused by the next tile)
  }
}

template <int VPL, int WKG, int WKD>
static hipError_t launch_fused_t(const Decode1Args& a, int num_cus, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&decode1_fused_bf16<VPL, WKG, WKD>);
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0);
  if (e != hipSuccess) return e;
  const int g = std::max(1, std::min(4, per_cu)) * num_cus;
  Decode1Args arg = a;
  void* args[] = {&arg};
  return hipLaunchCooperativeKernel(fn, dim3(g), dim3(256), args, 0, s);
}

template <int VPL>
static hipError_t launch_fused_vpl(const Decode1Args& a, int num_cus, hipStream_t s) {
  const bool g4 = a.d >= kStreamSplitK, d4 = a.f >= kStreamSplitK;
  if (g4 && d4) return launch_fused_t<VPL, 4, 4>(a, num_cus, s);
  if (g4) return launch_fused_t<VPL, 4, 2>(a, num_cus, s);
  if (d4) return launch_fused_t<VPL, 2, 4>(a, num_cus, s);
  return launch_fused_t<VPL, 2, 2>(a, num_cus, s);
}

hipError_t launch_decode1_fused(const Decode1Args& a, int num_cus, hipStream_t s) {
  if (a.E <= 64) return launch_fused_vpl<1>(a, num_cus, s);
  if (a.E <= 128) return launch_fused_vpl<2>(a, num_cus, s);
  if (a.E <= 256) return launch_fused_vpl<4>(a, num_cus, s);
  return launch_fused_vpl<8>(a, num_cus, s);
}

template <int VPL>
static void launch_decode1_vpl(const Decode1Args& a, const SelectOut& o, int g, hipStream_t s) {
  if (stream_bn(a.d) == 16) decode1_gate_up_bf16<VPL, 4><<<g, 256, 0, s>>>(a, o);
  else decode1_gate_up_bf16<VPL, 2><<<g, 256, 0, s>>>(a, o);
}

// Row-major weight bytes [rows][row_bytes] -> the tiled layout the streaming tiles of the narrow
// formats read: per 16-row block and chunk of cb bytes of a row (128 elements: cb = 64 for MXFP4,
// 128 for fp8), cb 16-byte units ordered [h < cb / 64][lane group g < 4][row r < 16], unit
// (h, g, r) = bytes [cb c + (cb / 4) g + 16 h, +16) of row 16 nb + r.  One unit per thread.
__global__ __launch_bounds__(256) void weight_tile_kernel(const uint8_t* __restrict__ src,
                                                          uint8_t* __restrict__ dst, int64_t rows,
                                                          int64_t row_bytes, int cb) {
  const int64_t nchunk = row_bytes / cb;
  const int64_t units = rows / 16 * nchunk * cb;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < units;
       t += (int64_t)gridDim.x * 256) {
    const int64_t blk = t / cb, u = t % cb;  // blk = nb * nchunk + c
    const int64_t nb = blk / nchunk, c = blk % nchunk;
    const int64_t h = u / 64, g = (u % 64) >> 4, r = u & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(src + (nb * 16 + r) * row_bytes + c * cb +
                                                    g * (cb / 4) + 16 * h);
    *reinterpret_cast<uint4*>(dst + t * 16) = v;
  }
}

hipError_t launch_weight_tile(const void* src, void* dst, int64_t rows, int64_t row_bytes, int cb,
                              hipStream_t s) {
  const int64_t units = rows / 16 * (row_bytes / cb) * cb;
  const int64_t grid = std::min<int64_t>((units + 255) / 256, 65536);
  if (grid > 0)
    weight_tile_kernel<<<(unsigned)grid, 256, 0, s>>>(static_cast<const uint8_t*>(src),
                                                      static_cast<uint8_t*>(dst), rows, row_bytes,
                                                      cb);
  return hipGetLastError();
}

hipError_t launch_decode1_bf16(const Decode1Args& a, const SelectOut& o, int num_cus,
                               hipStream_t s) {
  const int g = num_cus * 4;
  if (a.E <= 64) launch_decode1_vpl<1>(a, o, g, s);
  else if (a.E <= 128) launch_decode1_vpl<2>(a, o, g, s);
  else if (a.E <= 256) launch_decode1_vpl<4>(a, o, g, s);
  else launch_decode1_vpl<8>(a, o, g, s);
  return hipGetLastError();
}

template <bool GU>
static void launch_stream_bf16(const Seg* ss, int32_t* ms, int num_cus, int64_t max_rows,
                               int max_k, hipStream_t s, bool w4) {
  if (w4) {
    // passes of at most 32 rows: the 64-row pass needs 222 VGPRs (one wavefront per SIMD);
    // heavier experts take more passes (flushed: 1.075 -> 0.94 ms at T = 64, 1.63 -> 1.50 ms at
    // T = 256 on DeepSeek-V3-shaped layers).  Dynamic LDS: the staged scales of the workgroup's
    // weight rows (32 for K >= kStreamSplitK, else 64; gate and up) at a 256-byte-rounded stride.
    const size_t lds = (size_t)(GU ? 2 : 1) * (max_k >= kStreamSplitK ? 32 : 64) *
                       ((max_k / 32 + 255) / 256 * 256);
    if (max_rows <= 16) gemm_stream_bf16<GU, 1, true><<<num_cus * 4, 256, lds, s>>>(ss, ms);
    else gemm_stream_bf16<GU, 2, true><<<num_cus * 4, 256, lds, s>>>(ss, ms);
    return;
  }
  // Persistent grid: four workgroups per CU, six for one-row experts (the single-token down GEMM:
  // its 1792 tiles then take fewer uneven rounds, 51 -> 48 us on a DeepSeek-V3-shaped layer; at
  // T = 16 and 64 six were 1-3% slower)
  const int g = (max_rows <= 1 ? 6 : 4) * num_cus;
  if (GU && max_rows <= 1 && max_k <= kStreamXlMaxK)  // (down tiles are too short to gain)
    gemm_stream_bf16<GU, 0><<<g, 256, 0, s>>>(ss, ms);
  else if (max_rows <= 16) gemm_stream_bf16<GU, 1><<<g, 256, 0, s>>>(ss, ms);
  else if (max_rows <= 32) gemm_stream_bf16<GU, 2><<<g, 256, 0, s>>>(ss, ms);
  else gemm_stream_bf16<GU, 4><<<g, 256, 0, s>>>(ss, ms);
}

hipError_t launch_gemms_bf16(const SelectOut& o, int g, int num_cus, int64_t max_rows, int max_k,
                             bool stream, bool mfma, bool maybe_split, hipStream_t s, bool w4) {
  const Seg* ss = o.segs + (size_t)(g * kNumFam + kFamStream) * kSegCap;
  int32_t* ms = o.meta + (g * kNumFam + kFamStream) * kMetaStride;
  const Seg* sm = o.segs + (size_t)(g * kNumFam + kFamMfma) * kSegCap;
  int32_t* mm = o.meta + (g * kNumFam + kFamMfma) * kMetaStride;
  // split tiles: S >= 2 pieces each, all pieces within kSplitMaxPieces
  constexpr int kSplitGrid = kSplitMaxPieces / 2;
  const bool split = mfma && maybe_split && o.split_part;
  if (g == kGemmGateUp) {
    if (stream) launch_stream_bf16<true>(ss, ms, num_cus, max_rows, max_k, s, w4);
    if (mfma) gemm_mfma_bf16<true><<<num_cus, 256, 0, s>>>(sm, mm, o.split_part);
    if (split) mfma_split_epilogue<true><<<kSplitGrid, 256, 0, s>>>(sm, mm, o.split_part);
  } else {
    if (stream) launch_stream_bf16<false>(ss, ms, num_cus, max_rows, max_k, s, w4);
    if (mfma) gemm_mfma_bf16<false><<<num_cus, 256, 0, s>>>(sm, mm, o.split_part);
    if (split) mfma_split_epilogue<false><<<kSplitGrid, 256, 0, s>>>(sm, mm, o.split_part);
  }
  return hipGetLastError();
}

}  // namespace moe
