// Combine: gate-weighted gather-reduce back to token order (GC-MoE, summary: the combine step that
// follows the grouped GEMMs).  out[t] = bf16(sum_{j<k} w[t][j] * y[slot_dst[t*k+j]] (+ shared[t])),
// accumulated in fp32 in increasing j with the shared row last: deterministic, no atomics.
// Each thread owns 8 consecutive channels (16-byte loads and stores); a one-dimensional grid of
// T * nbx workgroups (token-major), so T is not bound by the grid's y limit.  The workgroup size is
// the largest of 256, 128 and 64 threads that divides a row's d / 8 threads, so no lane idles
// (d = 7168: 7 workgroups of 128 per token); y is read once, through non-temporal loads.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kCombineMaxThreads = 256;

__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ slot_dst,
                                                      const float* __restrict__ w, int k, int d,
                                                      int nbx, const uint16_t* __restrict__ sh,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x / nbx;
  const int c = ((blockIdx.x - t * nbx) * (int)blockDim.x + threadIdx.x) * 8;
  if (c >= d) return;
  // all k rows' indices and weights, then all k row loads, before any arithmetic (k <= 8)
  int row[kMaxTopK];
  float wj[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      row[j] = slot_dst[(size_t)t * k + j];
      wj[j] = w[(size_t)t * k + j];
    }
  }
  uint4 v[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j)
    if (j < k) {
      const u32x4 q = __builtin_nontemporal_load(
          reinterpret_cast<__attribute__((address_space(1))) const u32x4*>(
              (gchar*)(y + (size_t)row[j] * d + c)));
      v[j] = make_uint4(q.x, q.y, q.z, q.w);
    }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      const uint32_t p[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wj[j] * bf16_to_f32(uint16_t(p[i] & 0xFFFF));
        acc[2 * i + 1] += wj[j] * bf16_to_f32(uint16_t(p[i] >> 16));
      }
    }
  }
  if (sh) {
    const uint4 v = *reinterpret_cast<const uint4*>(sh + (size_t)t * d + c);
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += bf16_to_f32(uint16_t(p[i] & 0xFFFF));
      acc[2 * i + 1] += bf16_to_f32(uint16_t(p[i] >> 16));
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  *reinterpret_cast<uint4*>(out + (size_t)t * d + c) = o;
}

hipError_t launch_combine(const void* y, const int32_t* slot_dst, const float* w, int T, int k,
                          int d, const void* shared_y, void* out, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int lanes = d / 8;  // threads per token row
  const int bt = lanes % 256 == 0 ? 256 : lanes % 128 == 0 ? 128 : lanes % 64 == 0 ? 64 : 256;
  const int nbx = (lanes + bt - 1) / bt;
  combine_kernel<<<(unsigned)((int64_t)T * nbx), bt, 0, s>>>(static_cast<const uint16_t*>(y),
                                      slot_dst, w, k, d, nbx, static_cast<const uint16_t*>(shared_y),
                                      static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace moe
