// Per-token fp8 activation quantisation for block-scaled fp8 experts (GC-MoE, summary: FP8 grouped
// GEMM with requantisation).  Per token and per 128 channels: s = fp32(amax / 448) (s = 1 when amax
// is 0 or the quotient underflows), q = e4m3(fp32(x / s)).
//
// Both divisions go through float64 and are rounded once to float32: the exact quotient rounded to
// 53 bits and then to 24 bits equals the correctly rounded float32 quotient (53 >= 2*24 + 2), so the
// result does not depend on how the compiler lowers float division.
#include "common.h"
#include "kernels.h"
#include "fp8_codec.h"

namespace moe {

// One wavefront per (token, 128-channel group); each lane owns 2 channels.
__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t* __restrict__ x, int T,
                                                        int d, uint8_t* __restrict__ xq,
                                                        float* __restrict__ xs) {
  const int nb = d / 128;
  const int gidx = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gidx >= T * nb) return;
  const int lane = threadIdx.x & 63;
  const int t = gidx / nb, b = gidx % nb;
  const uint32_t pair = *reinterpret_cast<const uint32_t*>(x + (size_t)t * d + b * 128 + lane * 2);
  const float v0 = bf16_to_f32(uint16_t(pair & 0xFFFF)), v1 = bf16_to_f32(uint16_t(pair >> 16));
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float s = float(double(amax) / 448.0);
  if (amax == 0.0f || s == 0.0f) s = 1.0f;
  const uint8_t q0 = e4m3_encode(float(double(v0) / double(s)));
  const uint8_t q1 = e4m3_encode(float(double(v1) / double(s)));
  *reinterpret_cast<uint16_t*>(xq + (size_t)t * d + b * 128 + lane * 2) =
      uint16_t(q0) | (uint16_t(q1) << 8);
  if (lane == 0) xs[(size_t)t * nb + b] = s;
}

hipError_t launch_quant_act(const void* x, int T, int d, uint8_t* xq, float* xs, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int groups = T * (d / 128);
  quant_act_kernel<<<(groups + 3) / 4, 256, 0, s>>>(static_cast<const uint16_t*>(x), T, d, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
