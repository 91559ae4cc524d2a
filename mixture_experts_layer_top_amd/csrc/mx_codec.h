// MXFP8 block scales (E8M0) shared by the MXFP4 x MXFP8 tile kernels.
#pragma once

#include "common.h"

namespace moe {

// E8M0 scale code X = E + 127 of a block whose largest magnitude is amax (finite, >= 0): E is the
// smallest integer with amax <= 448 * 2^E, clamped to [-127, 127]; amax = 0 gives X = 127 (scale 1).
// With amax in [2^(e0 + 8), 2^(e0 + 9)), amax * 2^-e0 (amax's mantissa under the exponent of 256)
// lies in [256, 512) and E = e0 + 1 exactly when it exceeds 448.  Below 2^-126 E clamps to -127.
__device__ __forceinline__ int mx_scale_code(float amax) {
  if (amax == 0.0f) return 127;
  const uint32_t u = __float_as_uint(amax);
  const int ef = int(u >> 23);
  if (ef == 0) return 0;
  const int e0 = ef - 135;
  const float m = __uint_as_float((u & 0x7FFFFFu) | (135u << 23));
  const int e = e0 + (m > 448.0f ? 1 : 0);
  return max(e, -127) + 127;
}

// 2^-E for scale code X = E + 127 (E in [-127, 120]): the float with exponent field 254 - X.
__device__ __forceinline__ float mx_inv_scale(int X) { return __uint_as_float(uint32_t(254 - X) << 23); }

__device__ __forceinline__ void gstore_u8(uint8_t* p, size_t i, uint32_t v) {
  reinterpret_cast<__attribute__((address_space(1))) uint8_t*>((gwchar*)p)[i] = uint8_t(v);
}

}  // namespace moe
