// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// bf16 bit pattern <-> float (bf16 is the high half of an fp32).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Two fp32 -> packed bf16 (lo in the low half), round to nearest even: one v_cvt_pk_bf16_f32 on
// gfx950 (the same rounding as f32_to_bf16 for finite inputs).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// SiLU(g) * u in fp32, with the hardware exp2 and reciprocal (about 1 ulp each; the result is then
// rounded to bf16 or fp8).  g -> -inf gives exp -> inf, rcp -> 0 and the limit 0.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// MFMA wrappers.  Operand convention used throughout: the first operand ("A", MFMA rows i) holds
// weight rows, the second ("B", MFMA columns j) holds token rows; both are K-contiguous fragments.
//   16x16x32 bf16: lane l holds 8 bf16 of row/column (l % 16); C: lane l holds C[4*(l/16)+r][l%16].
//   32x32x16 bf16: lane l holds 8 bf16 of row/column (l % 32);
//                  C: lane l holds C[8*(r/4) + 4*(l/32) + r%4][l%32], r = 0..15.
//   16x16x128 fp8: lane l holds 32 e4m3 bytes of row/column (l % 16); C as 16x16x32.  In hardware
//                  lane group g = l / 16 holds K values 16 g .. + 15 and 64 + 16 g .. + 15 (an fp4
//                  operand: 32 g .. + 31); with unit E8M0 scales only the product matters, so two
//                  fp8 operands loaded alike (32 contiguous bytes at 32 g) still multiply correctly.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// fp8 x fp8 (both OCP e4m3, format code 0), unit E8M0 scales (127 = 2^0).
__device__ __forceinline__ f32x4 mfma16_fp8(const i32x8& a, const i32x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// Loads through the global address space (pointers read from memory are generic; flat loads would
// also count against the LDS wait counter and need 64-bit per-lane addresses).
typedef __attribute__((address_space(1))) const char gchar;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gload16(const void* base, uint32_t off) {
  const u32x4 v = *reinterpret_cast<__attribute__((address_space(1))) const u32x4*>((gchar*)base + off);
  return __builtin_bit_cast(uint4, v);
}
// The same with the non-temporal (streaming) cache policy, for weight bytes that one load reads
// whole (the tiled narrow-format layouts: 1 KB contiguous per wavefront) and nothing reads again.
// (Not for loads that take part of a 128-byte line each: evicted early, the line is fetched again
// for the rest -- the row-major bf16 streaming tile measured slower with it.)
__device__ __forceinline__ uint4 gload16_nt(const void* base, uint32_t off) {
  const u32x4 v = __builtin_nontemporal_load(
      reinterpret_cast<__attribute__((address_space(1))) const u32x4*>((gchar*)base + off));
  return __builtin_bit_cast(uint4, v);
}
__device__ __forceinline__ uint2 gload8(const void* base, uint32_t off) {
  const u32x2 v = *reinterpret_cast<__attribute__((address_space(1))) const u32x2*>((gchar*)base + off);
  return __builtin_bit_cast(uint2, v);
}
__device__ __forceinline__ uint32_t gload4(const void* base, uint32_t off) {
  return *reinterpret_cast<__attribute__((address_space(1))) const uint32_t*>((gchar*)base + off);
}
__device__ __forceinline__ uint32_t gload_u8(const uint8_t* p, uint32_t i) {
  return reinterpret_cast<__attribute__((address_space(1))) const uint8_t*>((gchar*)p)[i];
}
__device__ __forceinline__ int32_t gload_i32(const int32_t* p, int i) {
  return reinterpret_cast<__attribute__((address_space(1))) const int32_t*>((gchar*)p)[i];
}
__device__ __forceinline__ float gload_f32(const float* p, int i) {
  return reinterpret_cast<__attribute__((address_space(1))) const float*>((gchar*)p)[i];
}
// Vector stores through the global address space (a flat store would also count against the LDS
// wait counter, out of order, and force full waits on every LDS read behind it); off in bytes.
typedef __attribute__((address_space(1))) char gwchar;
__device__ __forceinline__ void gstore8(void* base, size_t off, uint2 v) {
  *reinterpret_cast<__attribute__((address_space(1))) u32x2*>((gwchar*)base + off) =
      __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ void gstore16(void* base, size_t off, uint4 v) {
  *reinterpret_cast<__attribute__((address_space(1))) u32x4*>((gwchar*)base + off) =
      __builtin_bit_cast(u32x4, v);
}
// The same with the non-temporal policy, for output that nothing reads again before it leaves the
// caches.
__device__ __forceinline__ void gstore16_nt(void* base, size_t off, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v),
                              reinterpret_cast<__attribute__((address_space(1))) u32x4*>((gwchar*)base + off));
}
__device__ __forceinline__ void gstore4(void* base, size_t off, uint32_t v) {
  *reinterpret_cast<__attribute__((address_space(1))) uint32_t*>((gwchar*)base + off) = v;
}
__device__ __forceinline__ void gstore_f32(float* p, size_t i, float v) {
  reinterpret_cast<__attribute__((address_space(1))) float*>((gwchar*)p)[i] = v;
}

// Device-coherent accesses (relaxed atomics at agent scope: global loads and stores with sc1): data
// written by one XCD and read by another within one kernel, whose L2s are not coherent.  The
// writer's stores are complete (acknowledged at the coherence point) once its vmcnt drains; a
// reader that then observes the writer's counter sees them with coherent loads.
__device__ __forceinline__ void gstore8_coh(void* base, size_t off, uint2 v) {
  const uint64_t x = ((uint64_t)v.y << 32) | v.x;
  __hip_atomic_store(reinterpret_cast<__attribute__((address_space(1))) uint64_t*>((gwchar*)base + off),
                     x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 gload8_coh(const void* base, size_t off) {
  const uint64_t x = __hip_atomic_load(
      reinterpret_cast<const __attribute__((address_space(1))) uint64_t*>((gchar*)base + off),
      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return uint2{(uint32_t)x, (uint32_t)(x >> 32)};
}
__device__ __forceinline__ int32_t counter_load(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t counter_add(int32_t* p, int32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void counter_store(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace moe
