// OCP E4M3FN encoder for the device (bias 7, 3 mantissa bits, largest finite 448, S.1111.111 = NaN,
// no infinities): round to nearest, ties to the even mantissa, saturate at +-448, keep the sign.
// Written from the format definition with integer operations only, so its rounding does not depend
// on a conversion instruction's modes.  Finite inputs only.  Host and device: the same source is
// compiled into a CPU harness that compares it with an independent encoder on every finite fp32
// bit pattern.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

__host__ __device__ __forceinline__ uint8_t e4m3_encode(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (u >> 31) << 7;
  const float a = __builtin_bit_cast(float, u & 0x7FFFFFFFu);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7E;
  } else if (a < 0.015625f) {  // below 2^-6: subnormal codes, steps of 2^-9
    // a * 512 is exact; round half to even to an integer in [0, 8] (8 = the smallest normal code)
    mag = uint32_t(__builtin_rintf(a * 512.0f));
  } else {
    const uint32_t ua = u & 0x7FFFFFFFu;
    const int e = int(ua >> 23) - 127;  // 2^-6 <= a < 448 -> e in [-6, 8]
    const uint32_t frac = ua & 0x7FFFFFu;
    uint32_t m = frac >> 20;
    const uint32_t rem = frac & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    uint32_t ef = uint32_t(e + 7);
    if (m == 8) {
      m = 0;
      ++ef;
    }
    mag = (ef << 3) | m;
    if (mag > 0x7E) mag = 0x7E;
  }
  return uint8_t(sign | mag);
}

}  // namespace moe
