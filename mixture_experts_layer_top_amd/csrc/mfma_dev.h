// Pieces shared by the LDS-staged MFMA tile kernels (bf16 and fp8): the direct global->LDS loads,
// explicit wait counts, and the per-XCD tile queues with their tile orders.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// The thread index through an opaque move: values the epilogues derive from it are computed there,
// instead of being hoisted out of the persistent tile loop and kept alive (or spilled) across the
// whole K loop.
__device__ __forceinline__ uint32_t tid_here() {
  uint32_t t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((uint32_t)threadIdx.x));
  return t;
}

// Epilogue of one tile: out is the GEMM's output base ([.][N] bf16), row0 + m0 its first row.

// A uniform value through an opaque scalar move (computations on it stay where they are written).
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with vmcnt(vm) and lgkmcnt(lg), expcnt left at its maximum (gfx9 encoding)
#define MOE_WAITCNT(vm, lg) \
  __builtin_amdgcn_s_waitcnt(((vm) & 15) | (((vm) >> 4) << 14) | 0x70 | (((lg) & 15) << 8))

// One global->LDS load of 16 bytes per lane: lane i's bytes land at dst + 16 * i (dst uniform).
// Written as asm because the compiler cannot tell which LDS bytes its LDS-load builtin writes: it
// waits for every such load (vmcnt(0)) before any LDS read that might overlap, which within one
// ring array means right after each prefetch is issued, and it also drains them at loop heads.  Hidden from the compiler, the loads still count in vmcnt in hardware, and vector
// memory operations of a wavefront complete in order; the short-tile pipeline waits for them
// explicitly, and any vmcnt wait the compiler emits for its own loads can only be stronger than
// needed.  No output registers: the data goes to LDS only.
// The address is a uniform 64-bit base in SGPRs plus the lane's 32-bit byte offset (the
// instruction's scalar-base form), so a lane keeps one offset register per load slot instead of a
// 64-bit address.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, lds_void* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  // (readfirstlane returns int: each half goes through uint32_t so that neither is sign-extended)
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(sb), "s"(lds)
               : "memory", "m0");
}

// The same for 4 bytes per lane: lane i's bytes land at dst + 4 * i.
__device__ __forceinline__ void dma4(const char* base, uint32_t off, lds_void* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(sb), "s"(lds)
               : "memory", "m0");
}

// Next tile for this workgroup from the per-XCD queues (see the scheduling note above), or -1.
// `q` is the workgroup's current queue offset (0 = its own XCD), kept across calls.
__device__ __forceinline__ int pop_tile_xcd(int32_t* queues, int ntiles, int chunk, int* slot,
                                            int& q) {
  const int xcd = blockIdx.x % kXcds;
  while (q < kXcds) {
    const int x = (xcd + q) % kXcds;
    if (threadIdx.x == 0) {
      const int i = atomicAdd(&queues[x], 1);
      *slot = (i / chunk) * (chunk * kXcds) + x * chunk + (i % chunk);
    }
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(*slot);
    __syncthreads();
    if (t < ntiles) return t;
    ++q;
  }
  return -1;
}

// Queue position -> tile index in the chunked order: class-0 tiles are [0, H) in tile order,
// class-1 ones [H, N).  Positions come in units of B (one XCD chunk); each class's whole units are
// spread evenly over the first U0 + U1 units (among the first u units, floor(u * U1 / U) are
// class 1), and the two classes' partial units (fewer than B tiles each) come last.
__device__ __forceinline__ int chunked_interleave(int p, int H, int N, int B) {
  const int L = N - H, U0 = H / B, U1 = L / B, U = U0 + U1;
  const int u = p / B, o = p - u * B;
  if (u < U) {
    const int c1 = (int)((long long)u * U1 / U), c1n = (int)((long long)(u + 1) * U1 / U);
    return c1n > c1 ? H + c1 * B + o : (u - c1) * B + o;
  }
  const int q = p - U * B, r0 = H - U0 * B;
  return q < r0 ? U0 * B + q : H + U1 * B + (q - r0);
}

// Queue position -> tile index in the mixed order: the L class-1 tiles spread evenly between the
// H class-0 ones (class-0 tiles are [0, H) in tile order, class-1 ones [H, H + L)): among the first
// p positions, floor(p * H / (H + L)) are class 0.  (32-bit products while they fit.)
__device__ __forceinline__ int interleave_tile(int p, int heavy, int ntiles) {
  int h0, h1;
  if (ntiles < 65536) {
    h0 = (int)((uint32_t)p * (uint32_t)heavy / (uint32_t)ntiles);
    h1 = (int)((uint32_t)(p + 1) * (uint32_t)heavy / (uint32_t)ntiles);
  } else {
    h0 = (int)(((long long)p * heavy) / ntiles);
    h1 = (int)(((long long)(p + 1) * heavy) / ntiles);
  }
  return h1 > h0 ? h0 : heavy + (p - h0);
}

}  // namespace moe
