// Host side of the C ABI declared in include/moe_mi355x.h: argument checks, workspace carving and
// kernel launches on the caller's stream.  No allocation, no synchronisation, no host reads of
// device data: every decision that depends on the routing is taken on the device.
#include "moe_mi355x.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>

#include "kernels.h"
#include "select_policy.h"

namespace {

using namespace moe;

static_assert(MOE_NUM_POLICIES == kNumPolicies, "the header's policy count");

constexpr size_t kAlign = 256;
constexpr int kMaxExperts = 512;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Sequential carving of a workspace (or a dry run that only sums the sizes when base is null).
struct Carver {
  uint8_t* base;
  size_t used = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align_up(count * sizeof(T));
    return p;
  }
};

// Compute units of the current device, queried on every call (the runtime answers from its cached
// device properties); the library keeps no state between calls.  0 if the query fails.
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n > 0 ? n : 0;
}

// The kernels address activation, h and y rows and one expert's weight matrix with 32-bit byte
// offsets (one VGPR per address instead of two): every such buffer must stay below 4 GiB.
constexpr int64_t kMaxOffsetBytes = int64_t(1) << 32;

int check_route_shape(int T, int E, int k) {
  if (T < 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (k > kMaxTopK || E > kMaxExperts || k > E) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool is_mxfp4(const moe_problem* p) {
  return p->wdtype == MOE_DTYPE_MXFP4 || p->wdtype == MOE_DTYPE_MXFP4_A8;
}

int check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  int st = check_route_shape(p->T, p->num_experts, p->top_k);
  if (st) return st;
  if (p->d_model <= 0 || p->d_ff <= 0) return MOE_ERR_INVALID_ARG;
  if (p->d_model % 128 || p->d_ff % 128) return MOE_ERR_UNSUPPORTED;
  if (p->wdtype != MOE_DTYPE_BF16 && p->wdtype != MOE_DTYPE_FP8_E4M3 &&
      p->wdtype != MOE_DTYPE_MXFP4 && p->wdtype != MOE_DTYPE_MXFP4_A8)
    return MOE_ERR_UNSUPPORTED;
  if (is_mxfp4(p) && p->has_shared) return MOE_ERR_UNSUPPORTED;
  // (MFMA tiles exist for mxfp4 weights with mxfp8 activations only)
  if (p->wdtype == MOE_DTYPE_MXFP4 && p->config == MOE_CONFIG_MFMA) return MOE_ERR_UNSUPPORTED;
  if (p->has_shared != 0 && p->has_shared != 1) return MOE_ERR_INVALID_ARG;
  if (p->has_shared && (p->d_ff_shared <= 0 || p->d_ff_shared % 128)) return MOE_ERR_UNSUPPORTED;
  const bool policy = p->config >= kConfigPolicy0 && p->config < kConfigPolicy0 + kNumPolicies;
  if ((p->config < MOE_CONFIG_AUTO || p->config > MOE_CONFIG_FUSED) && !policy)
    return MOE_ERR_INVALID_ARG;
  if (p->config == MOE_CONFIG_FUSED &&
      (p->T > 1 || p->wdtype != MOE_DTYPE_BF16 || p->has_shared || p->d_model > kStreamXlMaxK ||
       p->d_ff > kStreamXlMaxK))
    return MOE_ERR_UNSUPPORTED;
  if (policy && p->wdtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;  // (streaming only)
  // 32-bit byte offsets: x [T][d], h [T*k][f], y [T*k][d], shared h [T][f_sh] (2 bytes per value
  // at most) and each expert's [f][d] matrices must stay below 4 GiB
  const int64_t n = (int64_t)p->T * p->top_k;
  const int64_t f_sh = p->has_shared ? p->d_ff_shared : 0;
  const int64_t wide = std::max<int64_t>(std::max(p->d_model, p->d_ff), f_sh);
  if (n * wide * 2 >= kMaxOffsetBytes) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)p->d_model * std::max<int64_t>(p->d_ff, f_sh) * 2 >= kMaxOffsetBytes)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_weights(const moe_problem* p, const moe_weights* w, bool with_shared) {
  if (!w) return MOE_ERR_INVALID_ARG;
  // fp8 and mxfp4 weight bytes must be in the tiled layout (same size as the row-major one, so
  // the tag is the only thing that tells them apart); bf16 weights are row-major
  const int32_t want = p->wdtype == MOE_DTYPE_BF16 ? MOE_LAYOUT_ROW_MAJOR : MOE_LAYOUT_TILED;
  if (w->layout != want) return MOE_ERR_INVALID_ARG;
  const void* need[] = {w->w_gate, w->w_up, w->w_down};
  for (const void* q : need)
    if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (p->wdtype == MOE_DTYPE_FP8_E4M3) {
    if (!w->s_gate || !w->s_up || !w->s_down) return MOE_ERR_INVALID_ARG;
  }
  if (is_mxfp4(p)) {
    // (the tiles stage the scale rows with 4-byte loads)
    const void* e[] = {w->e_gate, w->e_up, w->e_down};
    for (const void* q : e)
      if (!q || reinterpret_cast<uintptr_t>(q) % 4) return MOE_ERR_INVALID_ARG;
  }
  if (with_shared && p->has_shared) {
    const void* sh[] = {w->sh_gate, w->sh_up, w->sh_down};
    for (const void* q : sh)
      if (!q || !aligned16(q)) return MOE_ERR_INVALID_ARG;
    if (p->wdtype == MOE_DTYPE_FP8_E4M3 && (!w->s_sh_gate || !w->s_sh_up || !w->s_sh_down))
      return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Workspace of the grouped GEMMs: segment lists, queue counters, the SwiGLU output and (bf16) the
// last-round split-K counters and partial sums.
struct FfnWs {
  Seg* segs;
  int32_t* meta;
  float* split_part;
  void* h;
  float* hs;
  uint8_t* he;
  uint8_t* xq;   // grouped FFN with MXFP8 activations: its own quantisation of x_perm
  uint8_t* xe;
  void* h_sh;
  float* hs_sh;
  void* y_sh;
};

// grouped_ffn: the grouped-FFN entry point (which quantises x_perm itself for MXFP8 activations)
void carve_ffn(Carver& c, const moe_problem* p, bool with_shared, bool grouped_ffn, FfnWs& f) {
  const size_t n = (size_t)p->T * p->top_k;
  const bool a8 = p->wdtype == MOE_DTYPE_MXFP4_A8;
  const size_t hb = (p->wdtype == MOE_DTYPE_FP8_E4M3 || a8) ? 1 : 2;  // bytes per h value
  f.segs = c.take<Seg>((size_t)2 * kNumFam * kSegCap);
  f.meta = c.take<int32_t>(2 * kNumFam * kMetaStride);
  f.split_part = nullptr;  // (only bf16 weights run MFMA tiles, which may split in K)
  if (p->wdtype == MOE_DTYPE_BF16)
    f.split_part = c.take<float>((size_t)kSplitMaxPieces * kSplitSlotFloats);
  f.h = c.take<uint8_t>(n * p->d_ff * hb);
  f.hs = p->wdtype == MOE_DTYPE_FP8_E4M3 ? c.take<float>(n * (p->d_ff / 128)) : nullptr;
  f.he = a8 ? c.take<uint8_t>(n * (p->d_ff / 32)) : nullptr;
  f.xq = f.xe = nullptr;
  if (a8 && grouped_ffn) {
    f.xq = c.take<uint8_t>(n * p->d_model);
    f.xe = c.take<uint8_t>(n * (p->d_model / 32));
  }
  f.h_sh = f.hs_sh = nullptr;
  f.y_sh = nullptr;
  if (with_shared && p->has_shared) {
    f.h_sh = c.take<uint8_t>((size_t)p->T * p->d_ff_shared * hb);
    f.hs_sh = hb == 1 ? c.take<float>((size_t)p->T * (p->d_ff_shared / 128)) : nullptr;
    f.y_sh = c.take<uint16_t>((size_t)p->T * p->d_model);
  }
}

// max_rows bounds the rows of any one expert and total_rows the rows of all of them.  The MFMA
// kernel (whose queue would be empty) is not launched when no expert can pass the streaming
// threshold, nor when the selection's few-tile rule must move every expert to the streaming tiles:
// no expert exceeds kFewTileRows rows and even one m-tile per expert that can hold rows would not
// make 1.6 rounds of CUs.  The split epilogue follows the MFMA kernel unless no list can split: a
// split needs fewer than kSplitMaxRounds rounds of MFMA tiles, and the MFMA rows are at least the
// rows of every expert above the streaming threshold, so when those alone fill kSplitMaxRounds
// rounds at full tile height no split can happen.
// The streaming thresholds of the policies the device may apply to a bf16 problem (the table row
// of its T bucket in automatic mode, else the forced one), and whether all of them use the few-tile
// rule: the host's launch decisions must hold for whichever one the live histogram picks.
struct PolicyBounds {
  int thr_min[2], thr_max[2];
  bool all_few;
};
PolicyBounds policy_bounds(const moe_problem* p) {
  PolicyBounds b{{1 << 30, 1 << 30}, {0, 0}, true};
  auto add = [&](int i) {
    const SelectPolicy& P = kPolicies[i];
    const int t[2] = {P.thr_gu, P.thr_dn};
    for (int g = 0; g < 2; ++g) {
      b.thr_min[g] = std::min(b.thr_min[g], t[g]);
      b.thr_max[g] = std::max(b.thr_max[g], t[g]);
    }
    b.all_few = b.all_few && P.few_tile;
  };
  if (p->config >= kConfigPolicy0) add(p->config - kConfigPolicy0);
  else
    for (int j = 0; j < kEeffBuckets; ++j) add(kPolicyTable[t_bucket(p->T)][j]);
  return b;
}

hipError_t launch_gemms(const SelectOut& o, const moe_problem* p, int gemm, int64_t max_rows,
                        int64_t total_rows, int cus, hipStream_t s) {
  if (p->wdtype == MOE_DTYPE_FP8_E4M3)
    return moe::launch_gemms_fp8(o, gemm, cus, max_rows, p->config != MOE_CONFIG_MFMA,
                                 p->config == MOE_CONFIG_MFMA ||
                                     (p->config == MOE_CONFIG_AUTO && max_rows > kFp8MfmaRows),
                                 s);
  if (p->wdtype == MOE_DTYPE_MXFP4_A8)
    return moe::launch_gemms_mx(o, gemm, cus, max_rows,
                                gemm == kGemmGateUp ? p->d_model : p->d_ff,
                                p->config != MOE_CONFIG_MFMA,
                                p->config == MOE_CONFIG_MFMA ||
                                    (p->config == MOE_CONFIG_AUTO && max_rows > kMxMfmaRows),
                                s);
  const int max_k_w4 = gemm == kGemmGateUp ? p->d_model : p->d_ff;
  if (p->wdtype == MOE_DTYPE_MXFP4)  // streaming tiles only
    return moe::launch_gemms_bf16(o, gemm, cus, max_rows, max_k_w4, true, false, false, s, true);
  const bool auto_mode = p->config == MOE_CONFIG_AUTO || p->config >= kConfigPolicy0;
  const PolicyBounds pb = policy_bounds(p);
  const bool stream = p->config != MOE_CONFIG_MFMA;
  bool mfma = p->config == MOE_CONFIG_MFMA || (auto_mode && max_rows > pb.thr_min[gemm]);
  const int64_t nt = gemm == kGemmGateUp ? p->d_ff / kMfmaBNGateUp
                                         : (p->d_model + kMfmaBNDown - 1) / kMfmaBNDown;
  if (mfma && auto_mode && pb.all_few && max_rows <= kFewTileRows && !p->has_shared) {
    const int64_t experts = std::min<int64_t>(p->num_experts, total_rows);
    if (5 * experts * nt < kFewTileRounds5 * (int64_t)cus) mfma = false;
  }
  const int64_t light = p->config == MOE_CONFIG_MFMA ? 0 : (int64_t)pb.thr_max[gemm] * p->num_experts;
  const int64_t min_tiles = (std::max<int64_t>(0, total_rows - light) + kMfmaBM - 1) / kMfmaBM * nt;
  const bool maybe_split =
      min_tiles < (int64_t)kSplitMaxRounds * std::min(cus, kSplitMaxPieces);
  const int max_k = gemm == kGemmGateUp ? p->d_model
                                         : std::max(p->d_ff, p->has_shared ? p->d_ff_shared : 0);
  return moe::launch_gemms_bf16(o, gemm, cus, max_rows, max_k, stream, mfma, maybe_split, s, false);
}
}  // namespace

extern "C" {

namespace {
int weight_tile(const void* src, void* dst, int64_t rows, int64_t cols, int bytes_per_128,
                hipStream_t stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || rows < 0 || cols < 0)
    return MOE_ERR_INVALID_ARG;
  if (rows % 16 || cols % 128) return MOE_ERR_UNSUPPORTED;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  const int64_t row_bytes = cols / 128 * bytes_per_128;
  const int64_t bytes = rows * row_bytes;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  return hip_status(moe::launch_weight_tile(src, dst, rows, row_bytes, bytes_per_128, stream));
}
}  // namespace

int moe_mxfp4_tile(const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t stream) {
  return weight_tile(src, dst, rows, cols, 64, stream);
}

int moe_fp8_tile(const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t stream) {
  return weight_tile(src, dst, rows, cols, 128, stream);
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null, misaligned or out-of-range argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or dtype outside the supported limits";
    case MOE_ERR_WORKSPACE:
      return "MOE_ERR_WORKSPACE: workspace missing or too small (moe_layer_noalloc: the problem "
             "needs more than the library's static scratch)";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch or runtime call failed";
    default: return "unknown moe status";
  }
}

int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
              hipStream_t stream) {
  int st = check_route_shape(T, E, k);
  if (st) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_route(logits, T, E, k, topk_ids, topk_w, stream));
}

size_t moe_permute_workspace_bytes(int T, int E, int k) {
  if (check_route_shape(T, E, k)) return 0;
  const size_t n = (size_t)T * k;
  Carver c{nullptr};
  c.take<int32_t>(n);
  c.take<int32_t>((size_t)permute_nchunk((int)n) * E);
  return c.used;
}

int moe_permute(const int32_t* topk_ids, int T, int E, int k, const void* x, const float* x_scale,
                int d, int act_dtype, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                int32_t* slot_dst, void* x_perm, float* x_perm_scale, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  int st = check_route_shape(T, E, k);
  if (st) return st;
  if (!counts || !offsets || !perm_src || !slot_dst) return MOE_ERR_INVALID_ARG;
  if (x_perm) {
    if (!x || d <= 0) return MOE_ERR_INVALID_ARG;
    if (d % 128) return MOE_ERR_UNSUPPORTED;
    if (act_dtype != MOE_DTYPE_BF16 && act_dtype != MOE_DTYPE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)T * k * (d / 128) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;  // scale index
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
    if (act_dtype == MOE_DTYPE_FP8_E4M3 && x_perm_scale && !x_scale) return MOE_ERR_INVALID_ARG;
  }
  if (T > 0 && !topk_ids) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_permute_workspace_bytes(T, E, k);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  const int n = T * k;
  Carver c{static_cast<uint8_t*>(ws)};
  int32_t* rank = c.take<int32_t>(n);
  int32_t* hist = c.take<int32_t>((size_t)permute_nchunk(n) * E);
  hipError_t e = launch_permute(topk_ids, T, E, k, counts, offsets, perm_src, slot_dst, nullptr,
                                rank, hist, stream);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (x_perm && n > 0) {
    const int fp8 = act_dtype == MOE_DTYPE_FP8_E4M3;
    e = launch_gather(x, fp8 ? x_scale : nullptr, perm_src, n, k, fp8 ? d : 2 * d, d / 128, x_perm,
                      fp8 ? x_perm_scale : nullptr, stream);
  }
  return hip_status(e);
}

int moe_quant_act_mx(const void* x, int T, int d, uint8_t* xq, uint8_t* xe, hipStream_t stream) {
  if (T < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
  if (d % 128) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * (d / 128) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;  // 32-bit group index
  if (T == 0) return MOE_OK;
  if (!x || !xq || !xe) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quant_act_mx(x, T, d, xq, xe, stream));
}

int moe_quant_act(const void* x, int T, int d, uint8_t* xq, float* xs, hipStream_t stream) {
  if (T < 0 || d <= 0) return MOE_ERR_INVALID_ARG;
  if (d % 128) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * (d / 128) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;  // 32-bit group index
  if (T == 0) return MOE_OK;
  if (!x || !xq || !xs) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quant_act(x, T, d, xq, xs, stream));
}

size_t moe_grouped_ffn_workspace_bytes(const moe_problem* p) {
  if (check_problem(p)) return 0;
  Carver c{nullptr};
  FfnWs f;
  carve_ffn(c, p, false, true, f);
  return c.used;
}

int moe_grouped_ffn(const moe_problem* p, const void* x_perm, const float* x_perm_scale,
                    const int32_t* counts, const int32_t* offsets, const moe_weights* w,
                    void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_problem(p);
  if (st) return st;
  if (p->config == MOE_CONFIG_FUSED) return MOE_ERR_UNSUPPORTED;  // (a layer-only path)
  st = check_weights(p, w, false);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  const int fp8 = p->wdtype == MOE_DTYPE_FP8_E4M3;
  if (!x_perm || !counts || !offsets || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(y_perm)) return MOE_ERR_INVALID_ARG;
  if (fp8 && !x_perm_scale) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_grouped_ffn_workspace_bytes(p);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carver c{static_cast<uint8_t*>(ws)};
  FfnWs f;
  carve_ffn(c, p, false, true, f);
  const int cus = device_cus();
  if (cus == 0) return MOE_ERR_HIP;
  SelectArgs a;
  std::memset(&a, 0, sizeof(a));
  a.counts = counts;
  a.offsets = offsets;
  a.E = p->num_experts;
  a.T = p->T;
  a.k = p->top_k;
  a.d = p->d_model;
  a.f = p->d_ff;
  a.has_shared = 0;
  a.config = p->config;
  a.num_cus = cus;
  a.fp8 = fp8;
  a.w4 = is_mxfp4(p);
  a.mx8 = p->wdtype == MOE_DTYPE_MXFP4_A8;
  a.e_gate = w->e_gate; a.e_up = w->e_up; a.e_down = w->e_down;
  a.x = a.mx8 ? static_cast<const void*>(f.xq) : x_perm;
  a.xe = f.xq ? f.xe : nullptr;
  a.he = f.he;
  a.xs = fp8 ? x_perm_scale : nullptr;
  a.tok = nullptr;
  a.w_gate = w->w_gate; a.w_up = w->w_up; a.w_down = w->w_down;
  a.s_gate = w->s_gate; a.s_up = w->s_up; a.s_down = w->s_down;
  a.h = f.h; a.hs = f.hs;
  a.y = y_perm;
  SelectOut o{f.segs, f.meta, f.split_part};
  const int64_t n = (int64_t)p->T * p->top_k;
  hipError_t e = hipSuccess;
  if (a.mx8) e = launch_quant_act_mx(x_perm, (int)n, p->d_model, f.xq, f.xe, stream);
  if (e == hipSuccess) e = launch_select(a, o, stream);  // caller-given counts: any expert may hold all rows
  if (e == hipSuccess) e = launch_gemms(o, p, kGemmGateUp, n, n, cus, stream);
  if (e == hipSuccess) e = launch_gemms(o, p, kGemmDown, n, n, cus, stream);
  return hip_status(e);
}

int moe_combine(const void* y_perm, const int32_t* slot_dst, const float* topk_w, int T, int k,
                int d, const void* shared_y, void* out, hipStream_t stream) {
  if (T < 0 || k <= 0 || d <= 0) return MOE_ERR_INVALID_ARG;
  if (k > kMaxTopK || d % 128) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_perm || !slot_dst || !topk_w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(out) || (shared_y && !aligned16(shared_y)))
    return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(y_perm, slot_dst, topk_w, T, k, d, shared_y, out, stream));
}

// Workspace of the whole layer (see carve_layer for the order).
namespace {
struct LayerWs {
  int32_t *sync, *ids, *counts, *offsets, *perm_src, *slot_dst, *tok, *rank, *hist;
  float* w;
  uint8_t* xq;
  float* xs;
  uint8_t* xe;
  void* y;
  FfnWs ffn;
};

void carve_layer(Carver& c, const moe_problem* p, LayerWs& L) {
  const size_t n = (size_t)p->T * p->top_k;
  const int E = p->num_experts;
  // the fused single-token launch's counters come first, in every layer workspace, so that no
  // other layer call writes them
  L.sync = c.take<int32_t>(kFusedSyncInts);
  L.ids = c.take<int32_t>(n);
  L.w = c.take<float>(n);
  L.counts = c.take<int32_t>(E);
  L.offsets = c.take<int32_t>(E + 1);
  L.perm_src = c.take<int32_t>(n);
  L.slot_dst = c.take<int32_t>(n);
  L.tok = c.take<int32_t>(n);
  L.rank = c.take<int32_t>(n);
  L.hist = c.take<int32_t>((size_t)permute_nchunk((int)n) * E);
  L.xq = nullptr;
  L.xs = nullptr;
  L.xe = nullptr;
  if (p->wdtype == MOE_DTYPE_FP8_E4M3 || p->wdtype == MOE_DTYPE_MXFP4_A8)
    L.xq = c.take<uint8_t>((size_t)p->T * p->d_model);
  if (p->wdtype == MOE_DTYPE_FP8_E4M3) L.xs = c.take<float>((size_t)p->T * (p->d_model / 128));
  if (p->wdtype == MOE_DTYPE_MXFP4_A8) L.xe = c.take<uint8_t>((size_t)p->T * (p->d_model / 32));
  carve_ffn(c, p, true, false, L.ffn);
  L.y = c.take<uint16_t>(n * p->d_model);
}
}  // namespace

size_t moe_layer_workspace_bytes(const moe_problem* p) {
  if (check_problem(p)) return 0;
  Carver c{nullptr};
  LayerWs L;
  carve_layer(c, p, L);
  return c.used;
}

namespace {
int layer_impl(const moe_problem* p, const float* logits, const void* x, const moe_weights* w,
               void* out, const moe_routing* keep, void* ws, size_t ws_bytes, hipEvent_t* ev,
               hipStream_t stream) {
  int st = check_problem(p);
  if (st) return st;
  st = check_weights(p, w, true);
  if (st) return st;
  if (p->T == 0) return MOE_OK;
  if (!logits || !x || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  const size_t need = moe_layer_workspace_bytes(p);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  Carver c{static_cast<uint8_t*>(ws)};
  LayerWs L;
  carve_layer(c, p, L);
  const int T = p->T, E = p->num_experts, k = p->top_k, d = p->d_model;
  const int fp8 = p->wdtype == MOE_DTYPE_FP8_E4M3;
  const int cus = device_cus();
  if (cus == 0) return MOE_ERR_HIP;
  int32_t* ids = (keep && keep->topk_ids) ? keep->topk_ids : L.ids;
  float* wts = (keep && keep->topk_w) ? keep->topk_w : L.w;
  int32_t* counts = (keep && keep->counts) ? keep->counts : L.counts;
  int32_t* offsets = (keep && keep->offsets) ? keep->offsets : L.offsets;
  int32_t* perm_src = (keep && keep->perm_src) ? keep->perm_src : L.perm_src;
  int32_t* slot_dst = (keep && keep->slot_dst) ? keep->slot_dst : L.slot_dst;
  float* out_eeff = keep ? keep->eeff : nullptr;
  int32_t* out_policy = keep ? keep->policy : nullptr;

  auto mark = [&](int i) -> hipError_t {
    return (ev && ev[i]) ? hipEventRecord(ev[i], stream) : hipSuccess;
  };

  SelectArgs a;
  std::memset(&a, 0, sizeof(a));
  a.counts = counts;
  a.offsets = offsets;
  a.E = E;
  a.T = T;
  a.k = k;
  a.d = d;
  a.f = p->d_ff;
  a.f_sh = p->has_shared ? p->d_ff_shared : 0;
  a.has_shared = p->has_shared;
  a.config = p->config;
  a.num_cus = cus;
  a.fp8 = fp8;
  a.w4 = is_mxfp4(p);
  a.mx8 = p->wdtype == MOE_DTYPE_MXFP4_A8;
  a.e_gate = w->e_gate; a.e_up = w->e_up; a.e_down = w->e_down;
  a.x = (fp8 || a.mx8) ? static_cast<const void*>(L.xq) : x;
  a.xs = L.xs;
  a.xe = L.xe;
  a.he = L.ffn.he;
  a.tok = L.tok;
  a.w_gate = w->w_gate; a.w_up = w->w_up; a.w_down = w->w_down;
  a.s_gate = w->s_gate; a.s_up = w->s_up; a.s_down = w->s_down;
  a.sh_gate = w->sh_gate; a.sh_up = w->sh_up; a.sh_down = w->sh_down;
  a.s_sh_gate = w->s_sh_gate; a.s_sh_up = w->s_sh_up; a.s_sh_down = w->s_sh_down;
  a.h = L.ffn.h; a.hs = L.ffn.hs;
  a.h_sh = L.ffn.h_sh; a.hs_sh = L.ffn.hs_sh;
  a.y = L.y; a.y_sh = L.ffn.y_sh;
  a.out_eeff = out_eeff;
  a.out_policy = out_policy;
  SelectOut o{L.ffn.segs, L.ffn.meta, L.ffn.split_part};

  hipError_t e = mark(0);
  if (p->config == MOE_CONFIG_FUSED) {  // (check_problem admitted one bf16 token, no shared expert)
    Decode1Args da;
    std::memset(&da, 0, sizeof(da));
    da.logits = logits;
    da.E = E;
    da.k = k;
    da.d = d;
    da.f = p->d_ff;
    da.x = x;
    da.w_gate = w->w_gate;
    da.w_up = w->w_up;
    da.w_down = w->w_down;
    da.h = L.ffn.h;
    da.y = L.y;
    da.ids = ids;
    da.w = wts;
    da.counts = counts;
    da.offsets = offsets;
    da.perm_src = perm_src;
    da.slot_dst = slot_dst;
    da.tok = L.tok;
    da.sync = L.sync;
    da.out = out;
    for (int i = 1; i <= 6 && e == hipSuccess; ++i) e = mark(i);
    if (e == hipSuccess) e = launch_decode1_fused(da, cus, stream);
    if (e == hipSuccess) e = mark(7);
    return hip_status(e);
  }
  // a single bf16 token without a shared expert: routing runs inside the gate/up kernel, which
  // also writes the routing outputs and the down GEMM's segments (phases 1 to 4 are empty)
  const bool decode1 = T == 1 && p->wdtype == MOE_DTYPE_BF16 && !p->has_shared &&
                       p->config != MOE_CONFIG_MFMA &&
                       d <= kStreamXlMaxK;
  if (decode1) {
    Decode1Args da;
    da.logits = logits;
    da.E = E;
    da.k = k;
    da.d = d;
    da.f = p->d_ff;
    da.x = x;
    da.w_gate = w->w_gate;
    da.w_up = w->w_up;
    da.w_down = w->w_down;
    da.h = L.ffn.h;
    da.y = L.y;
    da.ids = ids;
    da.w = wts;
    da.counts = counts;
    da.offsets = offsets;
    da.perm_src = perm_src;
    da.slot_dst = slot_dst;
    da.tok = L.tok;
    for (int i = 1; i <= 4 && e == hipSuccess; ++i) e = mark(i);
    if (e == hipSuccess) e = launch_decode1_bf16(da, o, cus, stream);
  } else if (front_small_fits(T, k)) {
    // decode-sized: route, permute and select in one launch (phases 1, 2 and 4 share it)
    if (e == hipSuccess)
      e = launch_front_small(logits, T, E, k, ids, wts, counts, offsets, perm_src, slot_dst,
                             L.tok, a, o, stream);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess && fp8) e = launch_quant_act(x, T, d, L.xq, L.xs, stream);
    if (e == hipSuccess && a.mx8) e = launch_quant_act_mx(x, T, d, L.xq, L.xe, stream);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = mark(4);
  } else {
    if (e == hipSuccess) e = launch_route(logits, T, E, k, ids, wts, stream);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess)
      e = launch_permute(ids, T, E, k, counts, offsets, perm_src, slot_dst, L.tok, L.rank,
                         L.hist, stream);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess && fp8) e = launch_quant_act(x, T, d, L.xq, L.xs, stream);
    if (e == hipSuccess && a.mx8) e = launch_quant_act_mx(x, T, d, L.xq, L.xe, stream);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = launch_select(a, o, stream);
    if (e == hipSuccess) e = mark(4);
  }
  // each token routes to k distinct experts, so no expert (nor the shared one) holds more than T rows
  if (e == hipSuccess && !decode1)
    e = launch_gemms(o, p, kGemmGateUp, T, (int64_t)T * p->top_k, cus, stream);
  if (e == hipSuccess) e = mark(5);
  if (e == hipSuccess) e = launch_gemms(o, p, kGemmDown, T, (int64_t)T * p->top_k, cus, stream);
  if (e == hipSuccess) e = mark(6);
  if (e == hipSuccess)
    e = launch_combine(L.y, slot_dst, wts, T, k, d, p->has_shared ? L.ffn.y_sh : nullptr, out,
                       stream);
  if (e == hipSuccess) e = mark(7);
  return hip_status(e);
}
}  // namespace

int moe_layer(const moe_problem* p, const float* logits, const void* x, const moe_weights* w,
              void* out, const moe_routing* keep, void* ws, size_t ws_bytes, hipStream_t stream) {
  return layer_impl(p, logits, x, w, out, keep, ws, ws_bytes, nullptr, stream);
}

int moe_layer_traced(const moe_problem* p, const float* logits, const void* x,
                     const moe_weights* w, void* out, const moe_routing* keep, void* ws,
                     size_t ws_bytes, hipEvent_t* events, int num_events, hipStream_t stream) {
  if (!events || num_events != MOE_TRACE_EVENTS) return MOE_ERR_INVALID_ARG;
  return layer_impl(p, logits, x, w, out, keep, ws, ws_bytes, events, stream);
}

}  // extern "C"
