// Tile-family selection for one workgroup (used by the selection kernel and the fused decode front
// end).  See select.hip for the policy.
#pragma once

#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {

constexpr int kSelMax = kSegCap;

__device__ __forceinline__ int pick_family(int c, int config, int fp8) {
  if (c <= 0) return -1;
  if (fp8) return kFamStream;  // block-scaled fp8 experts: streaming family only
  if (config == 0) return kFamStream;
  if (config >= 1) return kFamMfma;
  return c <= kStreamMaxRows ? kFamStream : kFamMfma;
}

// Per expert (one thread each, blockDim.x = 1024 >= E + 1): family, tile counts, and the segment's
// place in its family's list.  Order inside a family: experts with two or more m-tiles first
// ("heavy first", so the persistent queues start with the longest work), then by expert id; the
// ranks and tile bases come from one block-wide scan of 12 per-expert counts.  Every thread of the
// block must call this (it contains barriers).  Counts and offsets come from LDS when the caller
// has them there (lds_counts, lds_offsets), else from a.counts / a.offsets.
__device__ __forceinline__ void select_block(const SelectArgs& a, const SelectOut& o,
                                             const int* lds_counts = nullptr,
                                             const int* lds_offsets = nullptr) {
  __shared__ int scan_lds[16 * 12];
  const int e = threadIdx.x;
  const int nexp = a.E + (a.has_shared ? 1 : 0);
  int c = 0, fm = -1;
  if (e < nexp) {
    c = (e < a.E) ? (lds_counts ? lds_counts[e] : gload_i32(a.counts, e)) : a.T;
    fm = pick_family(c, a.config, a.fp8);
  }
  const bool shared = e == a.E;
  const int ffe = shared ? a.f_sh : a.f;
  const int tm = a.fp8 ? kStreamMaxRows8 : (fm == kFamStream) ? kStreamMaxRows : kMfmaBM;
  const int tn_gu = a.fp8 ? kStream8BNGateUp : (fm == kFamStream) ? stream_bn(a.d) : kMfmaBNGateUp;
  const int tn_dn = a.fp8 ? kStream8BNDown : (fm == kFamStream) ? stream_bn(ffe) : kMfmaBNDown;
  const int mtiles = (c + tm - 1) / tm;
  // f and d are multiples of 128; a down tile of 256 columns may be half full at the edge
  const int nt_gu = ffe / tn_gu, nt_dn = (a.d + tn_dn - 1) / tn_dn;
  const int cls = mtiles >= 2 ? 0 : 1;
  // v[4*f + 2*... ]: flags [fam][cls] (4), then tiles [gemm][fam][cls] (8)
  int v[12], ex[12], tot[12];
#pragma unroll
  for (int i = 0; i < 12; ++i) v[i] = 0;
  if (fm >= 0) {
    v[fm * 2 + cls] = 1;
    v[4 + (kGemmGateUp * 2 + fm) * 2 + cls] = mtiles * nt_gu;
    v[4 + (kGemmDown * 2 + fm) * 2 + cls] = mtiles * nt_dn;
  }
  block_scan<12, 16>(v, ex, tot, scan_lds);

  if (fm >= 0) {
    const int rank = (cls == 1 ? tot[fm * 2] : 0) + ex[fm * 2 + cls];
    const size_t wb = a.fp8 ? 1 : 2;
    const int row0 = shared ? 0 : (lds_offsets ? lds_offsets[e] : gload_i32(a.offsets, e));
    const int kb_d = a.d / 128, kb_f = ffe / 128;
    for (int g = 0; g < 2; ++g) {
      const int ti = 4 + (g * 2 + fm) * 2;
      Seg sg;
      sg.row0 = row0;
      sg.rows = c;
      sg.mtiles = mtiles;
      sg.expert = e;
      sg.tile_base = (cls == 1 ? tot[ti] : 0) + ex[ti + cls];
      sg.tn = (g == kGemmGateUp) ? tn_gu : tn_dn;
      if (g == kGemmGateUp) {
        sg.N = ffe;
        sg.K = a.d;
        sg.ntiles = nt_gu;
        sg.a = a.x;
        sg.as = a.xs;
        sg.tok = shared ? nullptr : a.tok;
        if (shared) {
          sg.w0 = a.sh_gate;
          sg.w1 = a.sh_up;
          sg.s0 = a.s_sh_gate;
          sg.s1 = a.s_sh_up;
          sg.out = a.h_sh;
          sg.outs = a.hs_sh;
        } else {
          const size_t wo = (size_t)e * ffe * a.d * wb;
          const size_t so = (size_t)e * kb_f * kb_d;
          sg.w0 = static_cast<const uint8_t*>(a.w_gate) + wo;
          sg.w1 = static_cast<const uint8_t*>(a.w_up) + wo;
          sg.s0 = a.s_gate ? a.s_gate + so : nullptr;
          sg.s1 = a.s_up ? a.s_up + so : nullptr;
          sg.out = a.h;
          sg.outs = a.hs;
        }
      } else {
        sg.N = a.d;
        sg.K = ffe;
        sg.ntiles = nt_dn;
        sg.tok = nullptr;
        sg.w1 = nullptr;
        sg.s1 = nullptr;
        sg.outs = nullptr;
        if (shared) {
          sg.a = a.h_sh;
          sg.as = a.hs_sh;
          sg.w0 = a.sh_down;
          sg.s0 = a.s_sh_down;
          sg.out = a.y_sh;
        } else {
          sg.a = a.h;
          sg.as = a.hs;
          sg.w0 = static_cast<const uint8_t*>(a.w_down) + (size_t)e * a.d * ffe * wb;
          sg.s0 = a.s_down ? a.s_down + (size_t)e * kb_d * kb_f : nullptr;
          sg.out = a.y;
        }
      }
      o.segs[((size_t)g * kNumFam + fm) * kSelMax + rank] = sg;
    }
  }
  // per (gemm, family): segment count, tile count, zeroed queues
  if (e < 2 * kNumFam) {
    const int g = e / kNumFam, f = e % kNumFam;
    o.meta[e * kMetaStride + 0] = tot[f * 2] + tot[f * 2 + 1];
    o.meta[e * kMetaStride + 1] = tot[4 + (g * 2 + f) * 2] + tot[4 + (g * 2 + f) * 2 + 1];
    for (int q = kMetaQueue; q < kMetaStride; ++q) o.meta[e * kMetaStride + q] = 0;
  }
}

}  // namespace moe
