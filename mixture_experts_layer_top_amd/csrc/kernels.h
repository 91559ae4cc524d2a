// Internal launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Tile families of the expert GEMMs.
enum Family { kFamStream = 0, kFamMfma = 1, kNumFam = 2 };
enum Gemm { kGemmGateUp = 0, kGemmDown = 1 };

constexpr int kMaxTopK = 8;  // experts per token (the boundary rejects more)

constexpr int kStreamMaxRows = 64;  // rows per weight-streaming pass
// Automatic selection: an expert takes the weight-streaming family for a GEMM while its row
// count is at most the policy's threshold for that GEMM (select_policy.h), the LDS-tiled MFMA
// family above it.
// Few-tile rule (policies that use it): a GEMM whose MFMA tiles would fill fewer than
// kFewTileRounds5 / 5 rounds of CUs runs wholly on the streaming tiles when none of its MFMA
// experts holds more than kFewTileRows rows (one 16-row MFMA pass per weight load); a larger
// expert keeps the whole GEMM on MFMA.
constexpr int kFewTileRows = 16;
constexpr int kFewTileRounds5 = 8;
constexpr int kMfmaBM = 256;        // rows per full LDS-tiled MFMA tile
constexpr int kMfmaBNGateUp = 128;  // h columns per gate/up MFMA tile (128 gate + 128 up rows)
constexpr int kMfmaBNDown = 256;    // y columns per down MFMA tile
constexpr int kXcds = 8;            // MI355X: 8 XCDs, each with its own L2
// Weight-streaming tiles: the 4 wavefronts split K four ways when K is long (16 output columns
// per tile), otherwise two ways (32 output columns, 16 per pair of wavefronts).  Measured: one
// wavefront per 16 columns over the whole K, or a four-way split of a short K, streams slower.
constexpr int kStreamSplitK = 4096;
__host__ __device__ constexpr int stream_bn(int K) { return K >= kStreamSplitK ? 16 : 32; }
// Longest K whose one-row activations a streaming tile stages in LDS (16 KB).
constexpr int kStreamXlMaxK = 8192;
constexpr int kSegCap = 1040;       // segment slots per (gemm, family); >= 2 * (E + 1)
// fp8 experts of more than kFp8MfmaRows rows take the LDS-staged MFMA tiles in automatic mode (when
// the GEMM's MFMA tiles fill at least one round of CUs), the others the streaming tiles.
constexpr int kFp8MfmaRows = 128;
// The same for mxfp4 experts with mxfp8 activations (whose streaming passes hold 32 rows).
constexpr int kMxMfmaRows = 64;
// fp8 weight-streaming tiles: rows per pass (more rows take more passes, which re-read
// the weights from L2; with 32 the down kernel fits three wavefronts per SIMD, while the gate/up
// kernel, which holds two K blocks of gate and up weights in flight, needs 256 VGPRs and runs one
// wavefront per SIMD), h columns per gate/up tile (one whole 128-column requantisation block), y
// columns per down tile
constexpr int kStreamMaxRows8 = 32;
constexpr int kStream8BNGateUp = 128;
constexpr int kStream8BNDown = 64;

// One expert's share of one grouped GEMM: out[row0 + r][n] for r < rows, n < N, from activation
// rows (gathered through `tok` when it is not null) and the expert's [N][K] weights.
struct Seg {
  const void* a;        // activation base ([.][K], bf16 or e4m3)
  const int32_t* tok;   // row -> activation row (null: row0 + r)
  const float* as;      // fp8: activation scales [.][K/128]
  const void* w0;       // gate (gate/up GEMM) or down weights, [N][K]
  const void* w1;       // up weights (gate/up GEMM), [N][K]
  const float* s0;      // fp8 block scales of w0, [N/128][K/128]
  const float* s1;      // fp8 block scales of w1
  const uint8_t* e0;    // mxfp4: E8M0 scales of w0, [N][K/32] (w0 then holds [N][K/2] bytes)
  const uint8_t* e1;    // mxfp4: E8M0 scales of w1
  const uint8_t* ae;    // mxfp8 activations: E8M0 scales [.][K/32] of the rows of `a`
  void* out;            // output base [.][N] (bf16, or e4m3 for the fp8 and mxfp8 gate/up GEMMs)
  float* outs;          // fp8 gate/up: output scales [.][N/128]
  uint8_t* oute;        // mxfp8 gate/up: output E8M0 scales [.][N/32]
  int32_t row0, rows, N, K;
  int32_t tile_base, mtiles, ntiles, expert;
  int32_t tn;           // output columns per tile
};

// Index of the segment holding tile t: the last one whose first tile (base[], in LDS) is <= t.
__device__ __forceinline__ int find_seg_lds(const int* base, int nseg, int t) {
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Last-round split of an MFMA GEMM: when its tiles leave a last round of CUs partly idle, the
// tiles of that round are split two or four ways in K, and every piece writes its fp32 partial sums
// to a slot of split_part.  A separate epilogue kernel, launched after the MFMA kernel, adds each
// split tile's slots in piece order (so results do not depend on which piece finished first) and
// stores the tile.
constexpr int kSplitMaxPieces = 256;  // partial-sum slots (one round of CUs)
constexpr int kSplitSlotFloats = 256 * 256;  // one full tile's accumulators
constexpr int kSplitMaxRounds = 3;    // longest-first order and split: fewer whole rounds than this
constexpr int kSplitMaxS = 4;         // pieces per split tile: 2 or 4

// Where the selection kernel writes its results (all inside the caller's workspace).
struct SelectOut {
  Seg* segs;           // [2 gemms][kNumFam][E + 1]
  int32_t* meta;       // [2 gemms][kNumFam][kMetaStride] (layout below)
  float* split_part;   // [kSplitMaxPieces][kSplitSlotFloats] partial sums (bf16 only, else null:
                       // no split; the two GEMMs run one after the other and share it)
};

// Everything the selection kernel needs to describe the two GEMMs.
struct SelectArgs {
  const int32_t* counts;   // [E]
  const int32_t* offsets;  // [E + 1]
  int E, T, k, d, f, f_sh, has_shared, config, fp8;
  int w4;                  // mxfp4 expert weights (streaming tiles)
  int mx8;                 // with mxfp8 activations (x and h quantised per 32; else bf16)
  const uint8_t* e_gate; const uint8_t* e_up; const uint8_t* e_down;  // their E8M0 scales
  const uint8_t* xe;       // mx8: E8M0 scales of the gate/up activations [.][d/32]
  uint8_t* he;             // mx8: E8M0 scales of h [T*k][f/32]
  int num_cus;              // compute units of the device (one MFMA-tile round)
  const void* x;           // gate/up activations (bf16 x, or e4m3 xq)
  const float* xs;         // fp8 activation scales
  const int32_t* tok;      // row -> token, for routed rows (null: rows are already permuted)
  const void* w_gate; const void* w_up; const void* w_down;
  const float* s_gate; const float* s_up; const float* s_down;
  const void* sh_gate; const void* sh_up; const void* sh_down;
  const float* s_sh_gate; const float* s_sh_up; const float* s_sh_down;
  void* h; float* hs;      // routed gate/up output [T*k][f] (+ fp8 scales [T*k][f/128])
  void* h_sh; float* hs_sh;  // shared gate/up output [T][f_sh]
  void* y; void* y_sh;     // down outputs [T*k][d], [T][d]
  float* out_eeff;         // optional: the live effective expert count (bf16 selection)
  int32_t* out_policy;     // optional: the policy the selection applied (-1: a family was forced)
};

// ints per (gemm, family): nseg, ntiles, then kXcds queue counters (the stream family uses the
// first), zeroed by the selection kernel before each GEMM, then the number of class-0 tiles (which
// come first in tile order; see select_dev.h), then (MFMA family) the first queue position whose
// tile is split in K and the pieces per split tile (positions [0, base) are whole tiles, and each
// tile of [base, ntiles) takes S consecutive positions), then the ordering mode, then kXcds more
// queue counters (the class-1 queues of the two-class order), also zeroed before each GEMM.
constexpr int kMetaStride = 32;
constexpr int kMetaQueue = 2;
constexpr int kMetaClass0 = kMetaQueue + kXcds;
constexpr int kMetaSplitBase = kMetaClass0 + 1;
constexpr int kMetaSplitS = kMetaClass0 + 2;
constexpr int kMetaOrder = kMetaClass0 + 3;  // tile order of an MFMA list (select_dev.h)
constexpr int kMetaQueue1 = kMetaOrder + 1;
enum TileOrder { kOrderMix = 0, kOrderTwoClass = 1, kOrderLongestFirst = 2 };
constexpr int kLongK = 4096;  // K from which an MFMA list takes the two-class order
static_assert(kMetaQueue1 + kXcds <= kMetaStride, "meta layout");
// Two-class order: relative CU time of a class-1 (short) tile against a class-0 (full-height) one,
// in twentieths, which sets how many of an XCD's CUs start on each class.
constexpr int kTwoClassW0 = 20, kTwoClassW1 = 11;

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s);
int permute_nchunk(int n);
hipError_t launch_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                          int32_t* offsets, int32_t* perm_src, int32_t* slot_dst, int32_t* tok,
                          int32_t* rank_ws, int32_t* hist_ws, hipStream_t s);
hipError_t launch_gather(const void* x, const float* xs, const int32_t* perm_src, int n, int k,
                         int row_bytes, int nb, void* xp, float* xps, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, const SelectOut& o, hipStream_t s);
// Decode front end (route + permute + select in one workgroup) when T*k <= 2048.
bool front_small_fits(int T, int k);
hipError_t launch_front_small(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                              int32_t* counts, int32_t* offsets, int32_t* perm_src,
                              int32_t* slot_dst, int32_t* tok, const SelectArgs& sa,
                              const SelectOut& so, hipStream_t s);
// Launches the persistent kernel of each tile family of one GEMM (kGemmGateUp or kGemmDown) that
// may hold tiles (the other's queue is empty).  max_rows bounds the rows of any one expert, max_k
// the GEMM's K over all its segments.
// Row-major weight bytes [rows][row_bytes] -> tiled layout in chunks of cb bytes per row
// (rows % 16 == 0, row_bytes % cb == 0; cb = 64 for MXFP4, 128 for fp8).
hipError_t launch_weight_tile(const void* src, void* dst, int64_t rows, int64_t row_bytes, int cb,
                              hipStream_t s);
// w4: mxfp4 weights (streaming tiles only; mfma must be false).  maybe_split: the MFMA list may
// hold tiles split in K (the host's bound), so the split epilogue kernel follows the MFMA kernel.
hipError_t launch_gemms_bf16(const SelectOut& o, int gemm, int num_cus, int64_t max_rows,
                             int max_k, bool stream, bool mfma, bool maybe_split, hipStream_t s,
                             bool w4);
// fp8: the streaming kernel and/or the LDS-staged MFMA kernel of one GEMM (each launched only when
// its list may hold tiles).
hipError_t launch_gemms_fp8(const SelectOut& o, int gemm, int num_cus, int64_t max_rows,
                            bool stream, bool mfma, hipStream_t s);
void launch_mfma_fp8(const Seg* segs, int32_t* meta, int gemm, int num_cus, hipStream_t s);
// MXFP4 weights with MXFP8 activations (streaming tiles on the scaled f8f6f4 MFMA); max_rows
// bounds any expert's rows, K is the GEMM's (d for gate/up, f for down).
hipError_t launch_gemms_mx(const SelectOut& o, int gemm, int num_cus, int64_t max_rows, int K,
                           bool stream, bool mfma, hipStream_t s);
void launch_mfma_mx(const Seg* segs, int32_t* meta, int gemm, int num_cus, hipStream_t s);
// x [T][d] bf16 -> MXFP8: xq [T][d] e4m3, xe [T][d/32] E8M0 (smallest scale with no saturation).
hipError_t launch_quant_act_mx(const void* x, int T, int d, uint8_t* xq, uint8_t* xe,
                               hipStream_t s);

// Single-token decode (T = 1, bf16 weights, no shared expert, d <= kStreamXlMaxK): one kernel routes
// the token in every workgroup (the k selected experts are then known without a dispatch step),
// runs the gate/up GEMM on streaming tiles, and from workgroup 0 writes the routing, the
// histogram, the permutation and the down GEMM's streaming segments, which the down kernel then
// takes as the selection kernel would have written them.
struct Decode1Args {
  const float* logits;  // [E]
  int E, k, d, f;
  const void* x;        // [d] bf16
  const void* w_gate; const void* w_up; const void* w_down;
  void* h;              // [k][f] bf16
  void* y;              // [k][d] bf16
  int32_t* ids; float* w;                 // [k]
  int32_t* counts; int32_t* offsets;      // [E], [E + 1]
  int32_t* perm_src; int32_t* slot_dst;   // [k]
  int32_t* tok;                           // [k]
  int32_t* sync;                          // fused launch: kFusedSyncInts counters (zero on entry)
  void* out;                              // fused launch: [d] bf16
};
constexpr int kFusedSyncInts = 9216;  // the fused single-token launch's counters (36 KB)
hipError_t launch_decode1_bf16(const Decode1Args& a, const SelectOut& o, int num_cus,
                               hipStream_t s);
// The whole single-token layer (routing, gate/up, down, combine) in one launch (MOE_CONFIG_FUSED;
// bf16, no shared expert, d and f <= kStreamXlMaxK).
hipError_t launch_decode1_fused(const Decode1Args& a, int num_cus, hipStream_t s);
hipError_t launch_combine(const void* y, const int32_t* slot_dst, const float* w, int T, int k,
                          int d, const void* shared_y, void* out, hipStream_t s);
hipError_t launch_quant_act(const void* x, int T, int d, uint8_t* xq, float* xs, hipStream_t s);

}  // namespace moe
