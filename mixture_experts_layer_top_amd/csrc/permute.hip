// Dispatch, single-GPU share: expert histogram, exclusive prefix sum, stable counting sort of the
// slots s = t*k + j into expert-contiguous rows, and the row gather.
//
// "Decoding the Skew ..." (Abstract) drives kernel choice from the live routing histogram; GC-MoE
// (summary) and Weave (Abstract) place token dispatch before the grouped GEMMs.  The layout here is
// unpadded: expert e owns rows [offsets[e], offsets[e+1]).
//
// Deterministic without float atomics and without a host sync:
//   count   : one workgroup per chunk of 2048 slots, processed as 8 rounds of 256 in slot order.
//             Inside a wavefront, lanes with the same expert are found with 9 ballots over the id
//             bits; a lane's rank is the popcount of equal lanes below it, plus the counts of the
//             earlier wavefronts and rounds of the chunk (LDS).  Writes rank[s] and the chunk's
//             histogram.
//   scan    : one workgroup; per expert, chunk histograms -> chunk base rows; counts; offsets.
//   scatter : row = chunk_base[chunk][e] + rank[s]; perm_src[row] = s; slot_dst[s] = row;
//             tok[row] = t (the activation row the GEMM gathers).
#include "common.h"
#include "kernels.h"
#include "route_dev.h"
#include "select_dev.h"

namespace moe {

constexpr int kChunk = 2048;
constexpr int kMaxE = 512;
constexpr int kScanBatch = 8;

__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ ids, int n,
                                                         int E, int32_t* __restrict__ rank,
                                                         int32_t* __restrict__ chunk_hist) {
  __shared__ int running[kMaxE];
  __shared__ int wcnt[4][kMaxE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int e = tid; e < E; e += 256) {
    running[e] = 0;
    wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
  }
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < kChunk / 256; ++r) {
    const int s = base + r * 256 + tid;
    const bool valid = s < n;
    const int e = valid ? ids[s] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank_w = __popcll(same & below);
    const int cnt_w = __popcll(same);
    const bool leader = valid && rank_w == 0;
    if (leader) wcnt[wv][e] = cnt_w;
    __syncthreads();
    if (valid) {
      int rk = running[e] + rank_w;
      for (int w = 0; w < wv; ++w) rk += wcnt[w][e];
      rank[s] = rk;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&running[e], cnt_w);
      wcnt[wv][e] = 0;
    }
    __syncthreads();
  }
  int32_t* hist = chunk_hist + (size_t)blockIdx.x * E;
  for (int e = tid; e < E; e += 256) hist[e] = running[e];
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t* __restrict__ chunk_hist,
                                                         int nchunk, int E, int n,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int tot[1024];
  const int e = threadIdx.x;
  int total = 0;
  // (chunks in batches of kScanBatch: the batch's loads go out together instead of one round trip
  // per chunk)
  if (e < E) {
    for (int c0 = 0; c0 < nchunk; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        h[i] = c0 + i < nchunk ? chunk_hist[(size_t)(c0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i) {
        if (c0 + i < nchunk) chunk_hist[(size_t)(c0 + i) * E + e] = total;
        total += h[i];
      }
    }
    counts[e] = total;
  }
  tot[e] = (e < E) ? total : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over 1024 entries.
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = (e >= off) ? tot[e - off] : 0;
    __syncthreads();
    tot[e] += v;
    __syncthreads();
  }
  if (e < E) {
    const int excl = tot[e] - total;
    offsets[e] = excl;
    for (int c0 = 0; c0 < nchunk; c0 += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (c0 + i < nchunk) h[i] = chunk_hist[(size_t)(c0 + i) * E + e];
#pragma unroll
      for (int i = 0; i < kScanBatch; ++i)
        if (c0 + i < nchunk) chunk_hist[(size_t)(c0 + i) * E + e] = h[i] + excl;
    }
  }
  if (e == 0) offsets[E] = n;
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids,
                                                           const int32_t* __restrict__ rank,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int n, int E, int k,
                                                           int32_t* __restrict__ perm_src,
                                                           int32_t* __restrict__ slot_dst,
                                                           int32_t* __restrict__ tok) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= n) return;
  const int e = ids[s];
  const int row = chunk_base[(size_t)(s / kChunk) * E + e] + rank[s];
  if (perm_src) perm_src[row] = s;
  if (slot_dst) slot_dst[s] = row;
  if (tok) tok[row] = s / k;
}

// x_perm[row] = x[tok[row]]: `bytes` per row, 16-byte vectors; one workgroup per 4 rows.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm_src,
                                                          int n, int k, int bytes,
                                                          uint8_t* __restrict__ xp) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int t = perm_src[row] / k;
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * bytes);
  uint4* dst = reinterpret_cast<uint4*>(xp + (size_t)row * bytes);
  for (int i = threadIdx.x & 63; i < bytes / 16; i += 64) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void gather_scales_kernel(const float* __restrict__ xs,
                                                            const int32_t* __restrict__ perm_src,
                                                            int n, int k, int nb,
                                                            float* __restrict__ xps) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n * nb) return;
  const int row = i / nb, b = i % nb;
  xps[i] = xs[(size_t)(perm_src[row] / k) * nb + b];
}

// ------------------------------------------------------------------------------------------------
// Decode front end: for T*k <= 2048, one workgroup of 1024 threads routes every token (one
// wavefront per token), ranks the slots stably inside LDS (two rounds of 1024, same ballot scheme
// as perm_count_kernel), scans the histogram, scatters the permutation and selects the tile
// families -- one launch instead of five.
// ------------------------------------------------------------------------------------------------
constexpr int kFrontMax = 2048;

template <int VPL>
__global__ __launch_bounds__(1024) void front_small_kernel(const float* __restrict__ logits, int T,
                                                           int E, int k, int32_t* __restrict__ ids,
                                                           float* __restrict__ w,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm_src,
                                                           int32_t* __restrict__ slot_dst,
                                                           int32_t* __restrict__ tok,
                                                           SelectArgs sa, SelectOut so) {
  __shared__ int s_ids[kFrontMax];
  __shared__ int wcnt[16][kMaxE];
  __shared__ int running[kMaxE];
  __shared__ int s_off[kMaxE];
  __shared__ int scan_lds[block_scan_lds(1)];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = T * k;
  for (int t = wv; t < T; t += 16) route_token<VPL>(logits, t, E, k, ids, w, s_ids);
  for (int e = tid; e < E; e += 1024) {
    running[e] = 0;
    for (int q = 0; q < 16; ++q) wcnt[q][e] = 0;
  }
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int myrank[2] = {0, 0}, myexp[2] = {0, 0};
  for (int r = 0; r * 1024 < n; ++r) {  // (n <= 2048; the bound is the same for every thread)
    const int s = r * 1024 + tid;
    const bool valid = s < n;
    const int e = valid ? s_ids[s] : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 9; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      same &= bit ? bb : ~bb;
    }
    const int rank_w = __popcll(same & below);
    const int cnt_w = __popcll(same);
    const bool leader = valid && rank_w == 0;
    if (leader) wcnt[wv][e] = cnt_w;
    __syncthreads();
    int rk = 0;
    if (valid) {
      rk = running[e] + rank_w;
      for (int q = 0; q < wv; ++q) rk += wcnt[q][e];
    }
    myrank[r] = rk;
    myexp[r] = e;
    __syncthreads();
    if (leader) {
      atomicAdd(&running[e], cnt_w);
      wcnt[wv][e] = 0;
    }
    __syncthreads();
  }
  // histogram scan (E <= 512 <= 1024 threads)
  int v[1], ex[1], tot[1];
  v[0] = tid < E ? running[tid] : 0;
  block_scan<1, 16>(v, ex, tot, scan_lds);
  if (tid < E) {
    s_off[tid] = ex[0];
    counts[tid] = v[0];
    offsets[tid] = ex[0];
  }
  if (tid == 0) offsets[E] = n;
  __syncthreads();
  for (int r = 0; r < 2; ++r) {
    const int s = r * 1024 + tid;
    if (s < n) {
      const int row = s_off[myexp[r]] + myrank[r];
      perm_src[row] = s;
      slot_dst[s] = row;
      tok[row] = s / k;
    }
  }
  __syncthreads();
  select_block(sa, so, running, s_off);
}

// One wavefront routes T/16 tokens one after the other, so the fused path only pays off while
// that is at most two tokens.
bool front_small_fits(int T, int k) { return T <= 32 && T * k <= kFrontMax; }

hipError_t launch_front_small(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                              int32_t* counts, int32_t* offsets, int32_t* perm_src,
                              int32_t* slot_dst, int32_t* tok, const SelectArgs& sa,
                              const SelectOut& so, hipStream_t s) {
  if (E <= 64)
    front_small_kernel<1><<<1, 1024, 0, s>>>(logits, T, E, k, ids, w, counts, offsets, perm_src,
                                             slot_dst, tok, sa, so);
  else if (E <= 128)
    front_small_kernel<2><<<1, 1024, 0, s>>>(logits, T, E, k, ids, w, counts, offsets, perm_src,
                                             slot_dst, tok, sa, so);
  else if (E <= 256)
    front_small_kernel<4><<<1, 1024, 0, s>>>(logits, T, E, k, ids, w, counts, offsets, perm_src,
                                             slot_dst, tok, sa, so);
  else
    front_small_kernel<8><<<1, 1024, 0, s>>>(logits, T, E, k, ids, w, counts, offsets, perm_src,
                                             slot_dst, tok, sa, so);
  return hipGetLastError();
}

int permute_nchunk(int n) { return (n + kChunk - 1) / kChunk; }

hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* perm_src, int32_t* slot_dst, int32_t* tok,
                          int32_t* rank_ws, int32_t* hist_ws, hipStream_t s) {
  const int n = T * k;
  const int nchunk = permute_nchunk(n);
  if (n > 0) perm_count_kernel<<<nchunk, 256, 0, s>>>(ids, n, E, rank_ws, hist_ws);
  perm_scan_kernel<<<1, 1024, 0, s>>>(hist_ws, nchunk, E, n, counts, offsets);
  if (n > 0)
    perm_scatter_kernel<<<(n + 255) / 256, 256, 0, s>>>(ids, rank_ws, hist_ws, n, E, k, perm_src,
                                                        slot_dst, tok);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const float* xs, const int32_t* perm_src, int n, int k,
                         int row_bytes, int nb, void* xp, float* xps, hipStream_t s) {
  if (n == 0) return hipSuccess;
  gather_rows_kernel<<<(n + 3) / 4, 256, 0, s>>>(static_cast<const uint8_t*>(x), perm_src, n, k,
                                                 row_bytes, static_cast<uint8_t*>(xp));
  if (xs && xps)
    gather_scales_kernel<<<(n * nb + 255) / 256, 256, 0, s>>>(xs, perm_src, n, k, nb, xps);
  return hipGetLastError();
}

}  // namespace moe
