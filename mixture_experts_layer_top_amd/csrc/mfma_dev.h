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
// NT: the non-temporal (streaming) cache policy, for bytes that no other tile reads.
template <bool NT = false>
__device__ __forceinline__ void dma16(const char* base, uint32_t off, lds_void* dst) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
  // (readfirstlane returns int: each half goes through uint32_t so that neither is sign-extended)
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | lo;
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off), "s"(sb), "s"(lds)
                 : "memory", "m0");
  else
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

// Next queue position for this workgroup from the per-XCD queues, or -1.  Workgroup b runs on XCD
// b % kXcds (the dispatcher deals workgroups to the XCDs in turn); queue x hands out the positions
// of XCD chunks x, x + kXcds, x + 2 kXcds, ... of `chunk` consecutive positions each, so the CUs of
// one XCD work on neighbouring tiles, which share weight and token tiles in its L2.  A workgroup
// drains its own XCD's queue, then takes from the others in turn.  `q` is the workgroup's current
// queue offset (0 = its own XCD), kept across calls.
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

// The two-class order: each XCD keeps one queue per class (class-0 tiles [0, n0) in tile order,
// class-1 tiles [n0, n0 + n1)), with XCD chunks of b0 class-0 and b1 class-1 positions.  Workgroups
// whose rank on their XCD (blockIdx.x / kXcds) is below r0 start on class 0, the others on class 1,
// so every XCD runs both classes at once: its full-height tiles, which all take the same K loop,
// stay in step in chunks that share operands in L2, while the short tiles stream beside them on
// the same XCD.  A workgroup drains its own class's queue on its XCD, then the other class's, then
// both queues of the other XCDs in turn.  Every position below a class's count is handed out
// exactly once: the positions of one queue grow with its counter, so a queue that returned one past
// its end is empty for good, and every workgroup visits every queue before it stops.  `q` counts
// the (XCD, class) queues this workgroup has finished; returns the tile index, or -1.
__device__ __forceinline__ int pop_tile_two_class(int32_t* queues0, int32_t* queues1, int n0, int n1,
                                                  int b0, int b1, int pref, int* slot, int& q) {
  const int xcd = blockIdx.x % kXcds;
  while (q < 2 * kXcds) {
    const int x = (xcd + (q >> 1)) % kXcds;
    const int c = (q & 1) ^ pref;
    const int b = c ? b1 : b0;
    if (threadIdx.x == 0) {
      const int i = atomicAdd(c ? &queues1[x] : &queues0[x], 1);
      *slot = (i / b) * (b * kXcds) + x * b + (i % b);
    }
    __syncthreads();
    const int p = __builtin_amdgcn_readfirstlane(*slot);
    __syncthreads();
    if (p < (c ? n1 : n0)) return c ? n0 + p : p;
    ++q;
  }
  return -1;
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
