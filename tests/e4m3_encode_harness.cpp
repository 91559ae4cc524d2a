// CPU harness for the library's E4M3 encoder (csrc/fp8_codec.h, host + device source): encodes a
// range of float32 bit patterns so that a test can compare every finite pattern with the oracle's
// independent codec.  Test infrastructure; built by tests/test_codec_exhaustive.py with hipcc
// --cuda-host-only (no GPU code).
#include <stdint.h>

#include "fp8_codec.h"

extern "C" void e4m3_encode_range(uint32_t start, uint32_t count, uint8_t* out) {
  for (uint32_t i = 0; i < count; ++i) out[i] = moe::e4m3_encode(__builtin_bit_cast(float, start + i));
}
