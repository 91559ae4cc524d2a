// Tile-family selection for one workgroup (used by the selection kernel and the fused decode front
// end).  See select.hip for the policy.
#pragma once

#include "common.h"
#include "kernels.h"
#include "route_dev.h"
#include "select_policy.h"

namespace moe {

constexpr int kSelThreads = 1024;  // one thread per expert (E + 1 <= kSelThreads)
static_assert(kSegCap >= 2 * (kSelThreads / 2 + 1), "two segments per expert (E <= 512)");

// config: -1 or a forced policy (>= kConfigPolicy0): the policy's thresholds; 0 / 1: that family.
// mxfp4 experts with bf16 activations stream; fp8 experts, and mxfp4 experts with mxfp8
// activations, take the MFMA tiles in automatic mode above kFp8MfmaRows / kMxMfmaRows rows (subject
// to the one-round check in select_block).
__device__ __forceinline__ int pick_family(int c, int g, int config, int fp8, int w4, int mx8,
                                           const SelectPolicy& P) {
  if (c <= 0) return -1;
  if (w4 && !mx8) return kFamStream;
  if (config == 0) return kFamStream;
  if (config == 1) return kFamMfma;
  if (fp8) return c > kFp8MfmaRows ? kFamMfma : kFamStream;
  if (mx8) return c > kMxMfmaRows ? kFamMfma : kFamStream;
  return c <= (g == kGemmGateUp ? P.thr_gu : P.thr_dn) ? kFamStream : kFamMfma;
}

// The live effective expert count exp(-sum_e q_e ln q_e), q_e = c_e / N, N = sum_e c_e, as
// exp(ln N - (sum_e c_e ln c_e) / N): one value per thread (c, 0 past the experts), summed in a
// fixed order (wavefront butterflies, then the wavefront totals in order).  Every thread of the
// block must call it; all get the result.
__device__ __forceinline__ float block_eeff(int c, int N) {
  __shared__ float part[kSelThreads / 64];
  float v = c > 1 ? (float)c * logf((float)c) : 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float S = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) S += part[w];
  __syncthreads();  // (part may be reused by the next call)
  return N > 0 ? expf(logf((float)N) - S / (float)N) : 0.f;
}

// Per expert (one thread each, blockDim.x = kSelThreads >= E + 1) and per GEMM: family, tile
// counts, and the segments' places in their (GEMM, family) list.  Each list has two classes of
// segments, class 0 first, each class by expert id, and the MFMA kernel hands its tiles out in one
// of three orders (kMetaOrder):
//  * kOrderMix (several rounds, short K or no expert of two m-tiles): class 0 = experts with two
//    or more m-tiles ("heavy"), class 1 = the rest; the light tiles are spread evenly between the
//    heavy ones, and an expert's last m-tile stays next to its siblings, which share its weight
//    tile in L2.  (Streaming lists use the same classes.)
//  * kOrderTwoClass (K >= kLongK, several rounds, some expert of more than one m-tile -- without one
//    no weight tile is shared by several m-tiles and the mixed order is faster, 3.5% on a
//    DeepSeek-V3-shaped layer at T = 256): an expert whose last 256-row m-tile would hold at most
//    128 rows gets that tail as a segment of its own; class 0 = segments of full-height tiles,
//    class 1 = shorter ones.  Every XCD keeps one queue per class (pop_tile_two_class): part of its
//    CUs runs the full-height tiles, which all take the same K loop, in chunks whose tiles stay in
//    step and share weight and token tiles in L2 (with long K, a short tile among them drifts its
//    neighbours apart: twice the gate/up L2 miss traffic was measured), while the rest streams the
//    short tiles beside them on the same XCD.  It replaced an order of whole XCD chunks of one
//    class each, which left an XCD on short tiles alone at times, their weight stream then limited
//    by that XCD's share of the fabric: gate/up 1.2% faster on a Mixtral-shaped layer and 1.5% on
//    a Kimi-K2-shaped one.  (Short K keeps the mixed order: the two-class order measured 5% slower
//    on the Kimi-K2-shaped down GEMM, K = 2048.)
//  * kOrderLongestFirst (one to kSplitMaxRounds rounds): classes as for kOrderTwoClass, tiles in
//    order -- round quantization dominates, so the short ones fill the last round, whose tiles may
//    be split in K.
// The ranks and tile bases come from one block-wide scan of 16 per-expert counts.  Every thread of
// the block must call this (it contains barriers).  Counts and offsets come from LDS when the
// caller has them there (lds_counts, lds_offsets), else from a.counts / a.offsets.
__device__ __forceinline__ void select_block(const SelectArgs& a, const SelectOut& o,
                                             const int* lds_counts = nullptr,
                                             const int* lds_offsets = nullptr) {
  __shared__ int scan_lds[block_scan_lds(16)];
  const int e = threadIdx.x;
  const int nexp = a.E + (a.has_shared ? 1 : 0);
  int c = 0;
  if (e < nexp) c = (e < a.E) ? (lds_counts ? lds_counts[e] : gload_i32(a.counts, e)) : a.T;
  const bool shared = e == a.E;
  const int ffe = shared ? a.f_sh : a.f;
  // The policy ("Decoding the Skew", Abstract: the live histogram matched to offline-tuned
  // configurations): bf16 problems in automatic mode look it up by T and the live effective expert
  // count; config >= kConfigPolicy0 forces one; forced families (config 0 / 1) and the streaming-only
  // formats use none.
  const bool bf16 = !a.fp8 && !a.w4;
  const float eeff = bf16 ? block_eeff(e < a.E ? c : 0, a.T * a.k) : 0.f;
  const bool auto_mode = a.config < 0 || a.config >= kConfigPolicy0;
  const int pol = !bf16 || !auto_mode ? -1
                  : a.config >= kConfigPolicy0 ? a.config - kConfigPolicy0
                                               : kPolicyTable[t_bucket(a.T)][eeff_bucket(eeff)];
  const SelectPolicy P = kPolicies[pol < 0 ? 0 : pol];
  if (e == 0) {
    if (a.out_eeff) a.out_eeff[0] = eeff;
    if (a.out_policy) a.out_policy[0] = pol;
  }
  int fm[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
    fm[g] = e < nexp ? pick_family(c, g, a.config, a.fp8, a.w4, a.mx8, P) : -1;
  // The down GEMM's light experts (<= kStreamRowsDown rows) take the streaming tiles only while its
  // heavier experts' MFMA tiles fill less than one round of CUs; with a round or more they join the
  // MFMA list, where their short tiles fill the rounds' gaps instead of running as a second launch
  // after the MFMA one (2-10% faster on DeepSeek-V3-shaped layers at T = 64 and 256 with 8 to 32
  // effective experts).
  // An MFMA tile costs a whole K loop on one CU, and one CU alone draws a fraction of the chip's
  // bandwidth, so a GEMM whose MFMA tiles would fill fewer than 1.6 rounds of CUs moves all its
  // experts to the streaming tiles, which spread each expert's weights over many workgroups -- but
  // only when every one of them is light (<= kFewTileRows rows).  With a heavier expert the GEMM
  // stays on MFMA: the streaming tiles lose to MFMA once an expert spans several 16-row passes, and
  // a split GEMM runs its two launches back to back with the MFMA one under-filled (1.3-1.5x the
  // all-MFMA time on a DeepSeek-V3-shaped layer at T = 64 and 256 with 8 effective experts).  The
  // same (block-wide) totals give the list's ordering mode: one to kSplitMaxRounds rounds ->
  // longest first (below one round every tile starts at once and order does not matter); else the
  // two-class order when K >= kLongK and some expert spans several m-tiles.
  // fp8 and mxfp8-activation experts (automatic mode): a GEMM whose MFMA tiles would fill less than
  // one round of CUs runs wholly on the streaming tiles (one CU per weight tile draws too little of
  // the chip's bandwidth).
  bool lpt[2] = {false, false}, two[2] = {false, false};
  if ((a.fp8 || a.mx8) && a.config < 0) {
    const int nt_dn = (a.d + kMfmaBNDown - 1) / kMfmaBNDown;
    int w[2], wex[2], wtot[2];
#pragma unroll
    for (int g = 0; g < 2; ++g)
      w[g] = fm[g] == kFamMfma
                 ? (c + kMfmaBM - 1) / kMfmaBM * (g == 0 ? ffe / kMfmaBNGateUp : nt_dn)
                 : 0;
    block_scan<2, 16>(w, wex, wtot, scan_lds);
#pragma unroll
    for (int g = 0; g < 2; ++g)
      if (fm[g] == kFamMfma && wtot[g] < a.num_cus) fm[g] = kFamStream;
  }
  if (!a.fp8 && !a.w4) {
    // w[0..1]: MFMA tiles per GEMM; w[2..3]: MFMA experts of more than one m-tile per GEMM;
    // w[4..5]: MFMA experts of more than kFewTileRows rows per GEMM; w[6]: down tiles of the light
    // experts the threshold put on the streaming tiles (w[7] unused)
    const int nt_dn = (a.d + kMfmaBNDown - 1) / kMfmaBNDown;
    int w[8], wex[8], wtot[8];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      w[g] = fm[g] == kFamMfma
                 ? (c + kMfmaBM - 1) / kMfmaBM * (g == 0 ? ffe / kMfmaBNGateUp : nt_dn)
                 : 0;
      w[2 + g] = fm[g] == kFamMfma && c > kMfmaBM ? 1 : 0;
      w[4 + g] = fm[g] == kFamMfma && c > kFewTileRows ? 1 : 0;
    }
    // (streamed down experts hold at most P.thr_dn <= 64 < kMfmaBM rows: one m-tile each)
    w[6] = auto_mode && P.promote && fm[kGemmDown] == kFamStream ? nt_dn : 0;
    w[7] = 0;
    block_scan<8, 16>(w, wex, wtot, scan_lds);
    if (auto_mode && P.promote && wtot[kGemmDown] >= a.num_cus) {
      if (w[6]) fm[kGemmDown] = kFamMfma;
      wtot[kGemmDown] += wtot[6];
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (auto_mode && P.few_tile && fm[g] == kFamMfma &&
          5 * wtot[g] < kFewTileRounds5 * a.num_cus && wtot[4 + g] == 0)
        fm[g] = kFamStream;
      const int C = min(a.num_cus, kSplitMaxPieces);
      lpt[g] = wtot[g] >= C && wtot[g] < kSplitMaxRounds * C;
      two[g] = !lpt[g] && (g == kGemmGateUp ? a.d : ffe) >= kLongK && wtot[2 + g] > 0;
    }
  }
  // Segment j = 2 * gemm + part (part 0: main, 1: MFMA tail), rows [r0[j], r0[j] + nr[j]) of the
  // expert; fam[j] < 0: no such segment.
  constexpr int NS = 4;
  const int tail = c > kMfmaBM && c % kMfmaBM <= kMfmaBM / 2 ? c % kMfmaBM : 0;
  int fam[NS], r0[NS], nr[NS], mt[NS], nt[NS], tn[NS], cls[NS];
  // v: flags [gemm][fam][cls] (8), then tiles [gemm][fam][cls] (8)
  int v[16], ex[16], tot[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) fam[j] = -1;
  // (threads past the experts skip the per-segment work; whole wavefronts of them branch over it)
  if (e < nexp) {
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int g = j >> 1, part = j & 1;
      const bool mf = fm[g] == kFamMfma;
      const bool split = mf && tail > 0 && (lpt[g] || two[g]);
      fam[j] = part == 0 ? fm[g] : (split ? kFamMfma : -1);
      r0[j] = part == 0 ? 0 : c - tail;
      nr[j] = part == 0 ? (split ? c - tail : c) : tail;
      const bool st = fam[j] == kFamStream;
      const int tm = st ? (a.fp8 ? kStreamMaxRows8 : kStreamMaxRows) : kMfmaBM;
      if (g == kGemmGateUp) {
        tn[j] = !st ? kMfmaBNGateUp : a.fp8 ? kStream8BNGateUp : (a.w4 ? 2 : 1) * stream_bn(a.d);
        nt[j] = ffe / tn[j];  // f is a multiple of 128
      } else {
        tn[j] = !st ? kMfmaBNDown : a.fp8 ? kStream8BNDown : (a.w4 ? 2 : 1) * stream_bn(ffe);
        // (a down tile of 256 columns may be half full at the edge)
        nt[j] = (a.d + tn[j] - 1) / tn[j];
      }
      mt[j] = (nr[j] + tm - 1) / tm;
      const bool by_height = mf && (lpt[g] || two[g]);
      cls[j] = by_height ? (nr[j] <= kMfmaBM / 2 ? 1 : 0) : (mt[j] >= 2 ? 0 : 1);
      // (all indexing below is static after unrolling, so nothing lands in scratch memory)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (fam[j] >= 0 && i == (g * 2 + fam[j]) * 2 + cls[j]) {
          v[i] += 1;
          v[8 + i] += mt[j] * nt[j];
        }
    }
  }
  block_scan<16, 16>(v, ex, tot, scan_lds);
  // (an expert's two segments of one GEMM have different classes, so each list index i takes at
  // most one segment per expert)
  int rank[NS], tbase[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int g = j >> 1;
    rank[j] = tbase[j] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (fam[j] >= 0 && i == (g * 2 + fam[j]) * 2 + cls[j]) {
        // class-1 segments follow all class-0 ones of their list
        rank[j] = ((i & 1) ? tot[i - 1] : 0) + ex[i];
        tbase[j] = ((i & 1) ? tot[8 + i - 1] : 0) + ex[8 + i];
      }
  }

  const size_t wb = a.fp8 ? 1 : 2;
  const int kb_d = a.d / 128, kb_f = ffe / 128;
  const int row0 = (e < nexp && !shared) ? (lds_offsets ? lds_offsets[e] : gload_i32(a.offsets, e)) : 0;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    if (fam[j] < 0) continue;  // (also every thread past the experts)
    const int g = j >> 1;
    Seg sg;
    sg.row0 = row0 + r0[j];
    sg.rows = nr[j];
    sg.mtiles = mt[j];
    sg.expert = e;
    sg.tile_base = tbase[j];
    sg.tn = tn[j];
    if (g == kGemmGateUp) {
      sg.N = ffe;
      sg.K = a.d;
      sg.ntiles = nt[j];
      sg.a = a.x;
      sg.as = a.xs;
      sg.tok = shared ? nullptr : a.tok;
      sg.ae = a.mx8 ? a.xe : nullptr;
      sg.oute = a.mx8 ? a.he : nullptr;
      if (shared) {
        sg.w0 = a.sh_gate;
        sg.w1 = a.sh_up;
        sg.e0 = sg.e1 = nullptr;
        sg.s0 = a.s_sh_gate;
        sg.s1 = a.s_sh_up;
        sg.out = a.h_sh;
        sg.outs = a.hs_sh;
      } else {
        const size_t wo = a.w4 ? (size_t)e * ffe * (a.d / 2) : (size_t)e * ffe * a.d * wb;
        const size_t eo = (size_t)e * ffe * (a.d / 32);
        sg.e0 = a.e_gate ? a.e_gate + eo : nullptr;
        sg.e1 = a.e_up ? a.e_up + eo : nullptr;
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
      sg.ntiles = nt[j];
      sg.tok = nullptr;
      sg.w1 = nullptr;
      sg.s1 = nullptr;
      sg.e1 = nullptr;
      sg.outs = nullptr;
      sg.ae = a.mx8 && !shared ? a.he : nullptr;
      sg.oute = nullptr;
      if (shared) {
        sg.a = a.h_sh;
        sg.as = a.hs_sh;
        sg.w0 = a.sh_down;
        sg.e0 = nullptr;
        sg.s0 = a.s_sh_down;
        sg.out = a.y_sh;
      } else {
        sg.a = a.h;
        sg.as = a.hs;
        sg.w0 = static_cast<const uint8_t*>(a.w_down) +
                (a.w4 ? (size_t)e * a.d * (ffe / 2) : (size_t)e * a.d * ffe * wb);
        sg.e0 = a.e_down ? a.e_down + (size_t)e * a.d * (ffe / 32) : nullptr;
        sg.s0 = a.s_down ? a.s_down + (size_t)e * kb_d * kb_f : nullptr;
        sg.out = a.y;
      }
    }
    o.segs[((size_t)g * kNumFam + fam[j]) * kSegCap + rank[j]] = sg;
  }
  // per (gemm, family): segment count, tile count, zeroed queues, class-0 tile count
  if (e < 2 * kNumFam) {  // e = gemm * kNumFam + family; its flags and tiles sit at 2e, 2e + 1
    int nseg = 0, ntl = 0, ntl0 = 0;
#pragma unroll
    for (int i = 0; i < 2 * kNumFam; ++i)
      if (i == e) {
        nseg = tot[2 * i] + tot[2 * i + 1];
        ntl = tot[8 + 2 * i] + tot[8 + 2 * i + 1];
        ntl0 = tot[8 + 2 * i];
      }
    int32_t* m = o.meta + e * kMetaStride;
    m[0] = nseg;
    m[1] = ntl;
    for (int q = kMetaQueue; q < kMetaQueue + kXcds; ++q) m[q] = 0;
    for (int q = kMetaQueue1; q < kMetaQueue1 + kXcds; ++q) m[q] = 0;
    m[kMetaClass0] = ntl0;
    // MFMA lists of bf16 GEMMs with fewer than kSplitMaxRounds whole rounds (longest first when
    // there is at least one) split in K the tiles past the last whole round of CUs, S = 4 or 2
    // ways, when their pieces still fit one round, every piece keeps an even number of 64-wide
    // K-steps, and K is the same for every segment.
    int base = ntl, S = 1;
    const int g = e / kNumFam;
    const int K = g == kGemmGateUp ? a.d : a.f;
    const bool uniform_k = g == kGemmGateUp || !a.has_shared || a.f_sh == a.f;
    const int C = min(a.num_cus, kSplitMaxPieces);
    const bool mfma_bf16 = e % kNumFam == kFamMfma && !a.fp8 && !a.w4;
    // (lpt[] is the same for every thread)
    m[kMetaOrder] = !mfma_bf16 ? kOrderMix : lpt[g] ? kOrderLongestFirst : two[g] ? kOrderTwoClass
                                                                                  : kOrderMix;
    if (mfma_bf16 && ntl < kSplitMaxRounds * C && o.split_part && uniform_k) {
      const int rounds = ntl / C, rem = ntl - rounds * C, nk = K / 64;
      if (rem > 0) {
        static_assert(kSplitMaxS == 4, "pieces per split tile");
        if (rem * 4 <= C && nk % 8 == 0) S = 4;
        else if (rem * 2 <= C && nk % 4 == 0) S = 2;
      }
      if (S > 1) base = ntl - rem;
    }
    m[kMetaSplitBase] = base;
    m[kMetaSplitS] = S;
  }
}

}  // namespace moe
