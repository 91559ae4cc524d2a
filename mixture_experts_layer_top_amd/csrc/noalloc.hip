// moe_layer_noalloc: the whole layer without a workspace argument, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The workspace moe_layer would take from the caller is a file-scope device array
// here, one copy per GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address comes
// from hipGetSymbolAddress, looked up once per device (with that device current) on the first call
// there and kept; only that address is ever passed to kernels.  The call then runs moe_layer's own
// kernels on it, so results are moe_layer's bit for bit.  Nothing here allocates, frees or
// synchronises.  Every call on one GPU shares that GPU's array, which keeps the last call's
// contents: the layer's kernels clear the counters and queues they need before use, and calls that
// overlap on one GPU (several streams or threads) race.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "moe_mi355x.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];

// This device's copy of `scratch` (nullptr if the lookup fails).
void* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);  // (two first calls store the same address)
  return p;
}

}  // namespace

extern "C" int moe_layer_noalloc(const moe_problem* p, const float* logits, const void* x,
                                 const moe_weights* w, void* out, const moe_routing* keep,
                                 hipStream_t stream) {
  const size_t need = moe_layer_workspace_bytes(p);  // 0: the problem itself is invalid
  if (need == 0) return moe_layer(p, logits, x, w, out, keep, nullptr, 0, stream);
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  if (p->T == 0) return moe_layer(p, logits, x, w, out, keep, nullptr, 0, stream);
  void* ws = device_scratch();
  if (!ws) return MOE_ERR_HIP;
  return moe_layer(p, logits, x, w, out, keep, ws, kScratchBytes, stream);
}
