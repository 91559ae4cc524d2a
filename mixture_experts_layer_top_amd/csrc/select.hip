// Device-side tile-configuration selection from the live routing histogram.
//
// "Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch" (Abstract):
// the best fused-MoE kernel changes with routing skew and token count, and static token-count
// buckets ignore the per-expert distribution that decides tile padding and memory reuse; the
// dispatch runtime reads the live histogram on the GPU, with no CPU-GPU synchronisation.
//
// Here the choice is made per expert, from its row count c_e, inside one workgroup that runs
// between the permutation and the GEMMs:
//   c_e <= 64  -> weight-streaming tiles: the expert's rows ride along while its weights stream
//                 from HBM once (decode-sized experts are bandwidth-bound: c_e FLOP per weight byte);
//   c_e  > 64  -> LDS-tiled MFMA tiles of 256 rows (padding only the last tile of the expert).
// Block-scaled fp8 experts always take the streaming family (up to 128 rows per pass).
// Experts of a family are ordered heaviest first (ties by id) so the persistent GEMM queues start
// with the longest work.  Experts with no rows get no segment and their weights are never read.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kSelMax = kSegCap;

__device__ __forceinline__ int pick_family(int c, int config, int fp8) {
  if (c <= 0) return -1;
  if (fp8) return kFamStream;  // block-scaled fp8 experts: streaming family only
  if (config == 0) return kFamStream;
  if (config >= 1) return kFamMfma;
  return c <= kStreamMaxRows ? kFamStream : kFamMfma;
}

__global__ __launch_bounds__(1024) void select_kernel(SelectArgs a, SelectOut o) {
  __shared__ int cnt[kSelMax];
  __shared__ int fam[kSelMax];
  __shared__ int scan[2][kNumFam][kSelMax];  // [gemm][family][rank] tiles, scanned in place
  const int e = threadIdx.x;
  const int nexp = a.E + (a.has_shared ? 1 : 0);
  int c = 0, fm = -1;
  if (e < nexp) {
    c = (e < a.E) ? a.counts[e] : a.T;
    fm = pick_family(c, a.config, a.fp8);
  }
  cnt[e] = c;
  fam[e] = fm;
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int f = 0; f < kNumFam; ++f) scan[g][f][e] = 0;
  __syncthreads();

  int rank = 0;
  if (fm >= 0)
    for (int q = 0; q < nexp; ++q)
      if (fam[q] == fm && (cnt[q] > c || (cnt[q] == c && q < e))) ++rank;

  const bool shared = e == a.E;
  const int ffe = shared ? a.f_sh : a.f;
  const int tm = a.fp8 ? kStreamMaxRows8 : (fm == kFamStream) ? kStreamMaxRows : kMfmaBM;
  const int tn_gu = a.fp8 ? kStream8BNGateUp : (fm == kFamStream) ? kStreamBN : kMfmaBNGateUp;
  const int tn_dn = a.fp8 ? kStream8BNDown : (fm == kFamStream) ? kStreamBN : kMfmaBNDown;
  const int mtiles = (c + tm - 1) / tm;
  // f and d are multiples of 128; a down tile of 256 columns may be half full at the edge
  const int nt_gu = ffe / tn_gu, nt_dn = (a.d + tn_dn - 1) / tn_dn;
  if (fm >= 0) {
    scan[kGemmGateUp][fm][rank] = mtiles * nt_gu;
    scan[kGemmDown][fm][rank] = mtiles * nt_dn;
  }
  __syncthreads();
  // inclusive Hillis-Steele scans of the four [rank] arrays
  for (int off = 1; off < kSelMax; off <<= 1) {
    int v[2][kNumFam];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int f = 0; f < kNumFam; ++f) v[g][f] = (e >= off) ? scan[g][f][e - off] : 0;
    __syncthreads();
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int f = 0; f < kNumFam; ++f) scan[g][f][e] += v[g][f];
    __syncthreads();
  }

  if (fm >= 0) {
    const size_t wb = a.fp8 ? 1 : 2;
    const int row0 = shared ? 0 : a.offsets[e];
    const int kb_d = a.d / 128, kb_f = ffe / 128;
    for (int g = 0; g < 2; ++g) {
      Seg sg;
      sg.row0 = row0;
      sg.rows = c;
      sg.mtiles = mtiles;
      sg.expert = e;
      const int own = (g == kGemmGateUp) ? mtiles * nt_gu : mtiles * nt_dn;
      sg.tile_base = scan[g][fm][rank] - own;
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
  // per (gemm, family): segment count, tile count, zeroed queue
  if (e < 2 * kNumFam) {
    const int g = e / kNumFam, f = e % kNumFam;
    int nseg = 0;
    for (int q = 0; q < nexp; ++q) nseg += (fam[q] == f);
    o.meta[e * kMetaStride + 0] = nseg;
    o.meta[e * kMetaStride + 1] = scan[g][f][kSelMax - 1];
    for (int q = kMetaQueue; q < kMetaStride; ++q) o.meta[e * kMetaStride + q] = 0;
  }
}

hipError_t launch_select(const SelectArgs& a, const SelectOut& o, hipStream_t s) {
  select_kernel<<<1, kSelMax, 0, s>>>(a, o);
  return hipGetLastError();
}

}  // namespace moe
