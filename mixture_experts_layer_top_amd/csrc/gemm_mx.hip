// MXFP4 expert weights with MXFP8 activations on gfx950's scaled matrix instruction.
//
// GC-MoE (summary) runs FP4 grouped GEMMs as block-scaled matrix multiplies, the FP4 weights decoded
// inside the matrix unit.  Here both operands are OCP microscaled: the weights are MXFP4 (E2M1
// pairs, one E8M0 scale per 32 along K, in the library's tiled layout) and the activations MXFP8
// (E4M3, one E8M0 scale per 32 channels, quantised by the layer with the smallest shared exponent
// E for which the block's largest magnitude is at most 448 * 2^E, so no element saturates).  One
// v_mfma_scale_f32_16x16x128_f8f6f4 multiplies 16 weight rows by 16 token rows over 128 K values
// and applies both sets of scales.  Lane l = 16 g + i covers weight row (or token) i; the K values
// it holds depend on the operand's format (found with a lane-layout probe of the instruction):
//   A, E2M1 (16 bytes): K values 32 g .. 32 g + 31, element 2j in the low nibble of byte j --
//      exactly the lane's 16-byte unit of the tiled weight layout;
//   B, E4M3 (32 bytes): K values 16 g .. 16 g + 15, then 64 + 16 g .. 64 + 16 g + 15;
//   scale_a / scale_b: lane 16 b + i carries the E8M0 byte of row (token) i and K block b (the
//      32 values 32 b .. 32 b + 31), whichever lanes hold those values.
// So weights go from HBM to the matrix unit with no conversion instruction, and activations stream
// at one byte per value instead of the W4A16 tile's two.
//
// Tiles follow the MXFP4 weight-streaming tile: a group of WK wavefronts covers 32 weight rows (two
// sets of 16) for up to 64 of an expert's rows, its wavefronts taking interleaved 128-value chunks
// of K, and the split-K partial sums meet in LDS in a fixed order.  The gate/up epilogue applies
// SwiGLU and requantises h to MXFP8 per token row and 32 columns -- the group's 32 columns are one
// block -- for the down GEMM, which reads h the same way and writes bf16.
#include "common.h"
#include "fp8_codec.h"
#include "kernels.h"
#include "mx_codec.h"
#include "mfma_dev.h"
#include "stream_dev.h"

namespace moe {

// ------------------------------------------------------------------------------------------------
// activation quantisation: x [T][d] bf16 -> xq [T][d] e4m3, xe [T][d/32] E8M0.  One wavefront per
// (token, 128 channels), two channels per lane, 16 lanes per block of 32.  x * 2^-E is exact in
// fp32 (a power-of-two scaling of a bf16 value whose magnitude ends at most 448) except where it
// falls below fp32's normal range, which E4M3 rounds to zero anyway.
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mx_quant_act_kernel(const uint16_t* __restrict__ x, int T,
                                                           int d, uint8_t* __restrict__ xq,
                                                           uint8_t* __restrict__ xe) {
  const int nb = d / 128;
  const int gidx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gidx >= T * nb) return;
  const int lane = threadIdx.x & 63;
  const int t = gidx / nb, b = gidx - t * nb;
  const size_t base = (size_t)t * d + b * 128 + lane * 2;
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(x + base);
  const float v0 = bf16_to_f32(uint16_t(pair & 0xFFFF)), v1 = bf16_to_f32(uint16_t(pair >> 16));
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const int X = mx_scale_code(amax);
  const float s = mx_inv_scale(X);
  const uint32_t q = uint32_t(e4m3_encode(v0 * s)) | (uint32_t(e4m3_encode(v1 * s)) << 8);
  *reinterpret_cast<uint16_t*>(xq + base) = uint16_t(q);
  if ((lane & 15) == 0) xe[(size_t)t * (d / 32) + b * 4 + (lane >> 4)] = uint8_t(X);
}

hipError_t launch_quant_act_mx(const void* x, int T, int d, uint8_t* xq, uint8_t* xe,
                               hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int groups = T * (d / 128);
  mx_quant_act_kernel<<<(groups + 3) / 4, 256, 0, s>>>(static_cast<const uint16_t*>(x), T, d, xq, xe);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// the streaming tile
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ i32x4 gload16i(const void* base, uint32_t off) {
  return __builtin_bit_cast(i32x4, gload16(base, off));
}
__device__ __forceinline__ i32x4 gload16i_nt(const void* base, uint32_t off) {
  return __builtin_bit_cast(i32x4, gload16_nt(base, off));
}

__device__ __forceinline__ f32x4 mfma_mx(const i32x4& w, uint32_t sw, const i32x8& x, uint32_t sx,
                                         const f32x4& c) {
  // A: E2M1 (format 4, only the first four dwords are read); B: E4M3 (format 0)
  const i32x8 a = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, x, c, 4, 0, 0, (int)sw, 0, (int)sx);
}

// One set's split-K reduction (every wavefront of the workgroup must call it): wavefronts kw > 0
// park their partials in LDS, wavefront kw = 0 adds them in kw order.
template <int MQ, int WK>
__device__ __forceinline__ void mx_reduce_set(float* red, int grp, int kw, f32x4 (&a0)[MQ],
                                              f32x4 (&a1)[MQ]) {
  if (WK == 1) return;
  const int lane = threadIdx.x & 63;
  constexpr int NV = MQ * 8;  // floats per lane (gate/up or one operand twice)
  __syncthreads();  // red[] may still be read
  if (kw > 0) {
    float* dst = red + ((grp * (WK - 1) + kw - 1) * NV) * 64 + lane;
#pragma unroll
    for (int q = 0; q < MQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dst[(q * 4 + i) * 64] = a0[q][i];
        dst[(MQ * 4 + q * 4 + i) * 64] = a1[q][i];
      }
  }
  __syncthreads();
  if (kw == 0) {
#pragma unroll
    for (int w = 0; w < WK - 1; ++w) {
      const float* src = red + ((grp * (WK - 1) + w) * NV) * 64 + lane;
#pragma unroll
      for (int q = 0; q < MQ; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a0[q][i] += src[(q * 4 + i) * 64];
          a1[q][i] += src[(MQ * 4 + q * 4 + i) * 64];
        }
    }
  }
}

// Gate/up epilogue of a group (wavefront kw = 0 after the reduction): h = SiLU(g) * u for 32
// columns n0 .. n0 + 31 and up to 16 * MQ rows, requantised to MXFP8 per row over the 32 columns.
// Lane (kg, r16) holds columns n0 + 16 h + 4 kg + i (h < 2, i < 4) of token column r16, so a
// row's block maximum is a maximum over the lane's 8 values and the 4 lanes kg = 0..3.
template <int MQ>
__device__ __forceinline__ void mx_gateup_store(const Seg& sg, int m0, int rows, int n0,
                                                const f32x4 (&g)[2][MQ], const f32x4 (&u)[2][MQ]) {
  const int lane = threadIdx.x & 63, r16 = lane & 15, kg = lane >> 4;
  const int N = sg.N;
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    float h[2][4];
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[s][i] = swiglu(g[s][q][i], u[s][q][i]);
        amax = fmaxf(amax, fabsf(h[s][i]));
      }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    const int X = mx_scale_code(amax);
    const float inv = mx_inv_scale(X);
    const int r = q * 16 + r16;
    if (r < rows) {
      const size_t orow = (size_t)(sg.row0 + m0 + r);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint32_t pk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) pk |= uint32_t(e4m3_encode(h[s][i] * inv)) << (8 * i);
        gstore4(sg.out, orow * N + n0 + 16 * s + 4 * kg, pk);
      }
      if (kg == 0) gstore_u8(sg.oute, orow * (N / 32) + n0 / 32, uint32_t(X));
    }
  }
}

// Stages the E8M0 scales a pass reads into LDS (sc): the workgroup's wrows weight rows from n0 (gate,
// then up), then the pass's 16 MQ token rows (padded rows as the first operand loads clamp them),
// KB bytes each at a row stride of RS = KB rounded up to 256 bytes.  Read per K block and lane from
// global memory instead, the scale bytes cost one load instruction touching 16 rows' cache lines
// per chunk and operand: with them the gate/up tile streamed at 54% of HBM on a DeepSeek-V3-shaped
// layer at T = 256, 79% in a timing build without them.  Each wavefront copies whole rows with
// direct global->LDS loads (a dword per lane, 256 bytes per instruction; lanes past the row re-read
// its last dword into the padding); the caller waits for them (vmcnt(0)) and holds a barrier
// before reading.  (The previous pass's reads of sc are behind the barriers of its split-K
// reduction.)
__device__ __forceinline__ int mx_scale_stride(int KB) { return (KB + 255) & ~255; }

template <int MQ, bool GU>
__device__ __forceinline__ void stage_scales_mx(const Seg& sg, int n0, int wrows, int KB,
                                                const int (&src)[MQ], uint8_t* sc) {
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int KW = KB / 4;  // dwords per row (K is a multiple of 128)
  const int RS = mx_scale_stride(KB);
  const int nw = (GU ? 2 : 1) * wrows, nrow = nw + 16 * MQ;
  for (int r = wv; r < nrow; r += 4) {
    const uint8_t* base;
    uint32_t row;
    if (r < nw) {
      base = GU && r >= wrows ? sg.e1 : sg.e0;
      row = (uint32_t)(n0 + (r < wrows ? r : r - wrows));
    } else {
      // token row t's source: lane t % 16 of src[t / 16] (uniform, so no per-row vector load --
      // whose wait would also wait for every staging load before it)
      const int t = r - nw;
      int v = src[0];
#pragma unroll
      for (int q = 1; q < MQ; ++q) v = t >= 16 * q ? src[q] : v;
      base = sg.ae;
      row = (uint32_t)__builtin_amdgcn_readlane(v, t & 15);
    }
    for (int i = 0; i < RS / 256; ++i) {
      const int c = min(64 * i + lane, KW - 1);
      dma4(reinterpret_cast<const char*>(base), row * (uint32_t)KB + 4 * c,
           (lds_void*)(sc + r * RS + 256 * i));
    }
  }
}

// Rows [m0, m0 + rows) (rows <= 16 * MQ) of segment sg, weight rows n0 + 32 grp .. + 31 of the
// calling group.  Wavefront kw takes the 128-value chunks kw, kw + WK, kw + 2 WK, ... of K.
template <int MQ, bool GU, int WK>
__device__ __forceinline__ void stream_tile_mx(const Seg& sg, int m0, int rows, int n0, float* red,
                                               uint8_t* sc) {
  constexpr int NR = 2;  // sets of 16 weight rows per group
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int K = sg.K, KB = K / 32;  // scale bytes per row
  const int grp = wv / WK, kw = wv % WK;
  const int wrows = 32 * (4 / WK);  // weight rows of the workgroup
  const int RS = mx_scale_stride(KB);
  const int n0wg = n0;
  n0 += 32 * grp;
  uint32_t wblk[NR], wsc[NR];  // this lane's unit in each set's 16-row block; its scale byte in LDS
#pragma unroll
  for (int s = 0; s < NR; ++s) {
    wblk[s] = (uint32_t)(n0 + 16 * s) * (uint32_t)(K / 2) + lane * 16;
    wsc[s] = (uint32_t)(32 * grp + 16 * s + r16) * (uint32_t)RS + kg;
  }
  const uint32_t wsc1 = (uint32_t)(wrows * RS);  // the up matrix's scales follow the gate's
  uint32_t xo[MQ], xso[MQ];  // this lane's activation bytes; its scale byte in LDS
  const uint32_t xs0 = (uint32_t)((GU ? 2 : 1) * wrows * RS);
  int src[MQ];
#pragma unroll
  for (int q = 0; q < MQ; ++q) {
    int r = q * 16 + r16;
    r = r < rows ? r : rows - 1;  // padded columns re-read a valid row; never stored
    const int gr = sg.row0 + m0 + r;
    src[q] = sg.tok ? gload_i32(sg.tok, gr) : gr;
    xo[q] = (uint32_t)src[q] * (uint32_t)K + kg * 16;  // B halves: bytes [16 kg, +16) and [64 + 16 kg, +16)
    xso[q] = xs0 + (uint32_t)(q * 16 + r16) * (uint32_t)RS + kg;
  }
  MOE_WAITCNT(0, 15);  // (the row gathers have landed: no wait behind the staging loads later)
  stage_scales_mx<MQ, GU>(sg, n0wg, wrows, KB, src, sc);
  f32x4 acc0[NR][MQ], acc1[NR][MQ];
#pragma unroll
  for (int s = 0; s < NR; ++s)
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      acc0[s][q] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1[s][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  // (a buffer holds the chunk's operands and its index; the scale bytes are read from LDS when the
  // chunk is computed)
  struct Blk { i32x4 w0[NR], w1[NR]; i32x8 x[MQ]; uint32_t c; };
  auto load = [&](Blk& b, int j) {
    const uint32_t c = (uint32_t)(j * WK + kw);
    b.c = c;
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      b.w0[s] = gload16i_nt(sg.w0, wblk[s] + c * 1024);
      if (GU) b.w1[s] = gload16i_nt(sg.w1, wblk[s] + c * 1024);
    }
#pragma unroll
    for (int q = 0; q < MQ; ++q) {
      const i32x4 lo = gload16i(sg.a, xo[q] + c * 128), hi = gload16i(sg.a, xo[q] + c * 128 + 64);
      b.x[q] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto compute = [&](const Blk& b) {
    const uint32_t c4 = 4 * b.c;
    uint32_t s0[NR], s1[NR], sx[MQ];
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      s0[s] = sc[wsc[s] + c4];
      if (GU) s1[s] = sc[wsc1 + wsc[s] + c4];
    }
#pragma unroll
    for (int q = 0; q < MQ; ++q) sx[q] = sc[xso[q] + c4];
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int q = 0; q < MQ; ++q) {
        acc0[s][q] = mfma_mx(b.w0[s], s0[s], b.x[q], sx[q], acc0[s][q]);
        if (GU) acc1[s][q] = mfma_mx(b.w1[s], s1[s], b.x[q], sx[q], acc1[s][q]);
      }
  };
  // The next two chunks' loads are in flight while a chunk is computed (three buffers, unrolled by
  // three; at the top of each round b0 and b1 hold chunks j and j + 1).  Scheduling barriers keep
  // each load group where it is written: hoisted above the computes, the later groups' loads sat
  // ahead of the chunk a compute waits for, and with in-order wait counts that wait drained them
  // too.  Loads past the wavefront's last chunk re-read that chunk (never computed), so the loop
  // body has no branch for the compiler to move the MFMAs across (with branches it also kept
  // duplicate buffers: 224 instead of 172 VGPRs).  Flushed, DeepSeek-V3-shaped, with the scales
  // staged in LDS: gate/up 0.827 -> 0.612 ms at T = 256 and 0.550 -> 0.458 ms at T = 64.
  const int nchunk = K / 128;
  const int nmine = (nchunk - kw + WK - 1) / WK;
  Blk b0, b1, b2;
  if (nmine > 0) load(b0, 0);
  if (nmine > 1) load(b1, 1);
  // (the first chunks' operand loads go out before the wait for the staged scales, so that their
  // latencies overlap)
  MOE_WAITCNT(0, 0);
  __syncthreads();
  int j = 0;
  for (; j + 3 <= nmine; j += 3) {
    load(b2, j + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(b0);
    __builtin_amdgcn_sched_barrier(0);
    load(b0, min(j + 3, nmine - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(b1);
    __builtin_amdgcn_sched_barrier(0);
    load(b1, min(j + 4, nmine - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(b2);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (j < nmine) compute(b0);
  if (j + 1 < nmine) compute(b1);
  if (GU) {
#pragma unroll
    for (int s = 0; s < NR; ++s) mx_reduce_set<MQ, WK>(red, grp, kw, acc0[s], acc1[s]);
    if (WK > 1 && kw != 0) return;
    mx_gateup_store<MQ>(sg, m0, rows, n0, acc0, acc1);
  } else {
    // (one reduction and bf16 epilogue per set; each ends with every wavefront past its barriers)
#pragma unroll
    for (int s = 0; s < NR; ++s)
      stream_tile_finish<MQ, false, WK>(sg, m0, rows, n0 + 16 * s, red, acc0[s], acc1[s]);
  }
}

// Rows [m0, m0 + rows) of a tile in passes of at most 16 * MQMAX rows (the host instantiates MQMAX
// from a bound on any expert's rows, which sets the kernel's register budget).
template <bool GU, int WK, int MQMAX>
__device__ __forceinline__ void stream_rows_mx(const Seg& sg, int m0, int rows, int n0, float* red,
                                               uint8_t* sc) {
  for (int sub = 0; sub < rows; sub += 16 * MQMAX) {
    const int r = min(16 * MQMAX, rows - sub);
    if (MQMAX == 1 || r <= 16) stream_tile_mx<1, GU, WK>(sg, m0 + sub, r, n0, red, sc);
    else if (MQMAX == 2 || r <= 32) stream_tile_mx<MQMAX >= 2 ? 2 : 1, GU, WK>(sg, m0 + sub, r, n0, red, sc);
    else stream_tile_mx<MQMAX, GU, WK>(sg, m0 + sub, r, n0, red, sc);
  }
}

// Persistent, as the other streaming kernels: workgroup b takes tile b first, then pops tiles
// gridDim.x, gridDim.x + 1, ... from the list's queue counter; segment bases are staged in LDS.
template <bool GU, int MQMAX>
__global__ __launch_bounds__(256) void gemm_stream_mx(const Seg* __restrict__ segs,
                                                       int32_t* __restrict__ meta) {
  __shared__ int slot;
  __shared__ int seg_base[kSegCap];
  __shared__ float red[3 * MQMAX * 8 * 64];
  extern __shared__ __attribute__((aligned(16))) uint8_t mx_sc[];  // staged scales (launch-sized)
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
    // long K: one group of 32 columns, 4-way split in K; else two groups of 32, wavefront pairs
    if (sg.tn == 32) stream_rows_mx<GU, 4, MQMAX>(sg, m0, rows, n0, red, mx_sc);
    else stream_rows_mx<GU, 2, MQMAX>(sg, m0, rows, n0, red, mx_sc);
    t = gridDim.x + __builtin_amdgcn_readfirstlane(pop_tile(&meta[kMetaQueue], &slot));
    if (t >= ntiles) break;
  }
}

// Passes of at most 32 rows: the 64-row pass needs 227 VGPRs, one wavefront per SIMD, and an
// expert of up to 64 rows is rare in decode; a heavier expert takes more passes over its weights
// (DeepSeek-V3-shaped, flushed: 1.065 -> 0.903 ms at T = 64 and 1.573 -> 1.348 ms at T = 256).
// Dynamic LDS of a launch: the staged scales of one pass (the GEMM's K is the same for every
// segment: no shared expert with mxfp4 weights).
constexpr size_t mx_scale_lds(bool gu, int K, int mq) {
  return (size_t)(((gu ? 2 : 1) * (K >= kStreamSplitK ? 32 : 64) + 16 * mq) *
                  ((K / 32 + 255) / 256 * 256));
}

template <bool GU>
static void launch_stream_mx(const Seg* ss, int32_t* ms, int num_cus, int64_t max_rows, int K,
                             hipStream_t s) {
  if (max_rows <= 16)
    gemm_stream_mx<GU, 1><<<num_cus * 4, 256, mx_scale_lds(GU, K, 1), s>>>(ss, ms);
  else
    gemm_stream_mx<GU, 2><<<num_cus * 4, 256, mx_scale_lds(GU, K, 2), s>>>(ss, ms);
}

hipError_t launch_gemms_mx(const SelectOut& o, int g, int num_cus, int64_t max_rows, int K,
                           bool stream, bool mfma, hipStream_t s) {
  const Seg* ss = o.segs + (size_t)(g * kNumFam + kFamStream) * kSegCap;
  int32_t* ms = o.meta + (g * kNumFam + kFamStream) * kMetaStride;
  if (stream) {
    if (g == kGemmGateUp) launch_stream_mx<true>(ss, ms, num_cus, max_rows, K, s);
    else launch_stream_mx<false>(ss, ms, num_cus, max_rows, K, s);
  }
  if (mfma)
    launch_mfma_mx(o.segs + (size_t)(g * kNumFam + kFamMfma) * kSegCap,
                   o.meta + (g * kNumFam + kFamMfma) * kMetaStride, g, num_cus, s);
  return hipGetLastError();
}

}  // namespace moe
