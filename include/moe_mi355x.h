/*
 * moe_mi355x.h -- C ABI of the fused MoE layer for one MI355X (gfx950).
 *
 * The layer (the pages describe it only step by step; the arithmetic below is the plainest
 * reading of a top-k softmax-routed SwiGLU MoE layer):
 *   route    per token, the k largest of E fp32 router logits (descending, ties to the lower expert
 *            id, -0.0 == +0.0) and their softmax renormalised over the selected k.  "Once routing
 *            completes, each layer's ... volumes become known" (Weave, Abstract).
 *   permute  expert histogram, exclusive prefix sum and a stable counting sort of the slots
 *            s = t*k + j into expert-contiguous rows: the single-GPU share of token dispatch
 *            (GC-MoE, summary; Weave, Abstract).
 *   experts  grouped gate/up GEMM with fused SwiGLU, then the grouped down GEMM, on shapes that
 *            follow the live routing histogram, chosen on the device with no host sync
 *            ("Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch",
 *            Abstract; GC-MoE, summary: fused SwiGLU, FP8 requantisation, optional shared experts).
 *   combine  out[t] = sum_j w[t,j] * y[slot_dst[t*k+j]] (+ shared[t]), summed in fp32 in j order,
 *            rounded once to bf16 (GC-MoE, summary: "combine step").
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller; the two structs are host memory
 *     read during the call only.  The library never allocates, frees or synchronises: every call
 *     only enqueues work on `stream` and returns; outputs are valid once the stream reaches them.
 *   - Layouts are row-major.  bf16 values are 16-bit bfloat16 bit patterns; fp8 values are OCP
 *     E4M3FN bytes (bias 7, max 448, S.1111.111 = NaN).
 *   - Expert weights are stored with the contraction dimension contiguous:
 *       w_gate, w_up [E][d_ff][d_model]   (math shape d_model x d_ff)
 *       w_down       [E][d_model][d_ff]   (math shape d_ff x d_model)
 *     fp8 weights carry one fp32 scale per 128x128 block: s_gate, s_up [E][d_ff/128][d_model/128],
 *     s_down [E][d_model/128][d_ff/128]; the weight's value is code * scale.  fp8 weight bytes
 *     (routed and shared) are passed in the library's tiled layout, made once by moe_fp8_tile
 *     from the row-major one; the block scales stay row-major.
 *     mxfp4 weights (OCP MX MXFP4; GC-MoE, summary: FP4 grouped GEMM decoded in registers) pack
 *     two E2M1 codes per byte, element 2j in the low nibble of byte j: w_gate, w_up
 *     [E][d_ff][d_model/2], w_down [E][d_model][d_ff/2] bytes, with one E8M0 scale byte X per 32
 *     elements along the contraction dimension: e_gate, e_up [E][d_ff][d_model/32], e_down
 *     [E][d_model][d_ff/32]; the weight's value is e2m1(code) * 2^(X - 127).  Scales must lie in
 *     [2, 252] (not checked), which keeps every scaled weight an exact bf16 value.  The weight
 *     bytes are passed in the library's tiled layout, made once by moe_mxfp4_tile from the
 *     row-major one; the scales stay row-major.
 *   - Return value: MOE_OK or an error code; moe_status_string() names it.  Arguments are checked
 *     on the host only (null pointers, sizes, 16-byte alignment, workspace size).  Device data is
 *     not validated: non-finite logits or out-of-range expert ids are undefined behaviour.
 *     T = 0 is a valid no-op.  A failed launch returns MOE_ERR_HIP.
 *   - Limits: 1 <= k <= 8, k <= E <= 512, d_model and d_ff multiples of 128, T*k < 2^31.  The
 *     kernels address rows with 32-bit byte offsets, so moe_layer and moe_grouped_ffn also need
 *     T*k*max(d_model, d_ff, d_ff_shared)*2 < 2^32 and d_model*max(d_ff, d_ff_shared)*2 < 2^32
 *     (every activation, h and y buffer and each expert matrix below 4 GiB); moe_quant_act needs
 *     T*d/128 < 2^31 and moe_permute's gather T*k*d/128 < 2^31.  Outside them: MOE_ERR_UNSUPPORTED.
 *   - Calls are reentrant: no mutable global state (the device's compute-unit count is queried on
 *     every call); concurrent calls need distinct workspaces.  The one exception is
 *     moe_layer_noalloc, whose workspace is a static per-GPU array (see its declaration).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2, /* shape or dtype outside the limits above */
  MOE_ERR_WORKSPACE = 3,   /* workspace null or smaller than the *_workspace_bytes() figure */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
};

enum moe_dtype {
  MOE_DTYPE_BF16 = 0,
  MOE_DTYPE_FP8_E4M3 = 1,
  MOE_DTYPE_MXFP4 = 2, /* expert weights only: bf16 activations, no shared expert, streaming tiles
                          only (config MOE_CONFIG_MFMA and has_shared give MOE_ERR_UNSUPPORTED).
                          e_gate, e_up and e_down must be 4-byte aligned */
  MOE_DTYPE_MXFP4_A8 = 3 /* MXFP4 expert weights with MXFP8 activations: the layer quantises x (and
                            the SwiGLU output h) per token and 32 channels to E4M3 with one E8M0
                            scale each (the smallest scale 2^E with amax <= 448 * 2^E), and both
                            GEMMs run on the scaled f8f6f4 MFMA.  No shared expert; e_* 4-byte
                            aligned; MOE_CONFIG_MFMA is supported (256 x 256 LDS-staged tiles) */
};

/* Tile configuration for the expert GEMMs.  MOE_CONFIG_AUTO lets the device pick per expert and per
 * GEMM from the live histogram: for bf16 weights it computes the histogram's effective expert count
 * (exp of its entropy) and looks up, by T and that count, a selection policy tuned offline ("Decoding
 * the Skew", Abstract: the live distribution matched to offline-tuned configurations).  The others
 * force one family for every expert, or (MOE_CONFIG_POLICY0 + i, bf16 only) force policy i; tests
 * use them to cover each.  Block-scaled fp8 weights in automatic mode put experts of more than 128
 * rows (mxfp4 weights with mxfp8 activations: more than 64) on the MFMA tiles when a GEMM's MFMA
 * tiles fill at least one round of compute units, the others on the streaming tiles (no policy
 * table); mxfp4 weights with bf16 activations always stream. */
enum moe_config {
  MOE_CONFIG_AUTO = -1,
  MOE_CONFIG_STREAM = 0, /* weight-streaming tiles: up to 64 of an expert's rows per pass */
  MOE_CONFIG_MFMA = 1,   /* LDS-tiled MFMA tiles: bf16 64, 128 or 256 rows (from the rows a tile
                            holds) x 256 weight rows; fp8 and mxfp4 with mxfp8 activations
                            256 x 256 (mxfp4 with bf16 activations: MOE_ERR_UNSUPPORTED) */
  MOE_CONFIG_FUSED = 2,  /* moe_layer of one bf16 token without a shared expert, d_model and d_ff
                            <= 8192: the whole layer in one launch ("Weave", Abstract:
                            an MoE layer as one persistent megakernel; GC-MoE, summary: a decode
                            step launched as one graph).  Every workgroup routes the token and
                            takes gate/up, then down tiles from a device queue; a down tile waits
                            for its row's gate/up tiles and the last down tile of each column
                            block combines it, through device counters that live
                            in the first 36 KB of the workspace.  Those 36 KB must be zero before
                            the first such call (zero the workspace once when allocating it);
                            every call leaves them zero, and no other call writes them.  A wait
                            that does not end within about a second sets the int at byte offset
                            32768 of the workspace and gives up (the output is then wrong).  Other
                            problems, and moe_grouped_ffn, give MOE_ERR_UNSUPPORTED */
  MOE_CONFIG_POLICY0 = 16 /* 16 + i (i < MOE_NUM_POLICIES): selection policy i, whatever the
                             histogram (other values: MOE_ERR_INVALID_ARG) */
};
#define MOE_NUM_POLICIES 8

typedef struct moe_problem {
  int32_t T;           /* tokens */
  int32_t d_model;     /* hidden size d */
  int32_t d_ff;        /* routed expert intermediate size f */
  int32_t num_experts; /* E */
  int32_t top_k;       /* k */
  int32_t wdtype;      /* enum moe_dtype of the expert weights (activations are bf16 at the boundary) */
  int32_t has_shared;  /* 1: one always-active shared SwiGLU expert, added with weight 1 */
  int32_t d_ff_shared; /* its intermediate size (multiple of 128) */
  int32_t config;      /* enum moe_config */
} moe_problem;

/* Storage layout of the expert weight bytes (moe_weights.layout).  bf16 weights are row-major; fp8
 * and mxfp4 weight bytes must be in the library's tiled layout, made by moe_fp8_tile /
 * moe_mxfp4_tile.  The two layouts have the same size, so the tag is what tells them apart: a
 * mismatch gives MOE_ERR_INVALID_ARG instead of silently wrong outputs. */
enum moe_layout {
  MOE_LAYOUT_ROW_MAJOR = 0,
  MOE_LAYOUT_TILED = 1
};

typedef struct moe_weights {
  const void* w_gate; /* [E][f][d] bf16 or e4m3 */
  const void* w_up;   /* [E][f][d] */
  const void* w_down; /* [E][d][f] */
  const float* s_gate; /* fp8 only: [E][f/128][d/128]; NULL for bf16 */
  const float* s_up;
  const float* s_down; /* [E][d/128][f/128] */
  const void* sh_gate; /* shared expert (has_shared), [f_sh][d], same dtype */
  const void* sh_up;
  const void* sh_down; /* [d][f_sh] */
  const float* s_sh_gate; /* fp8 only */
  const float* s_sh_up;
  const float* s_sh_down;
  const uint8_t* e_gate; /* mxfp4 only: E8M0 scales [E][f][d/32]; NULL otherwise */
  const uint8_t* e_up;
  const uint8_t* e_down; /* [E][d][f/32] */
  int32_t layout;        /* enum moe_layout of w_* and sh_*: MOE_LAYOUT_TILED for fp8 and mxfp4,
                            MOE_LAYOUT_ROW_MAJOR for bf16 */
} moe_weights;

/* Optional routing outputs of moe_layer (any member may be NULL to skip it). */
typedef struct moe_routing {
  int32_t* topk_ids; /* [T][k] */
  float* topk_w;     /* [T][k] */
  int32_t* counts;   /* [E] */
  int32_t* offsets;  /* [E+1] */
  int32_t* perm_src; /* [T*k] */
  int32_t* slot_dst; /* [T*k] */
  float* eeff;        /* [1]: the live effective expert count the bf16 selection computed */
  int32_t* policy;    /* [1]: the policy it applied (-1 when a family was forced); neither is
                         written for fp8 / mxfp4 weights or the single-token bf16 path */
} moe_routing;

/* Route: topk_ids[t][j] = j-th largest logit's expert (ties -> lower id), topk_w[t][j] = its
 * weight in the softmax renormalised over the selected k, computed in fp32 (expf of the gap to the
 * largest selected logit, divided by their sum).
 *   logits [T][E] fp32.  Outputs [T][k]. */
int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
              hipStream_t stream);

/* Permute (dispatch share): counts[e] = #slots routed to e; offsets[0..E] its exclusive prefix sum
 * (offsets[E] = T*k); perm_src[row] = slot s = t*k+j placed at expert-contiguous row `row`, in
 * increasing s inside each expert (stable); slot_dst[s] = row.  If x_perm is not NULL, also gathers
 * x_perm[row] = x[perm_src[row] / k]: act_dtype MOE_DTYPE_BF16 copies d bf16 values per row;
 * MOE_DTYPE_FP8_E4M3 copies d e4m3 bytes per row and, if x_perm_scale is not NULL, the d/128 fp32
 * scales per row from x_scale.
 *   topk_ids [T][k] int32 in [0, E).  ws: moe_permute_workspace_bytes(T, E, k) bytes. */
int moe_permute(const int32_t* topk_ids, int T, int E, int k, const void* x, const float* x_scale,
                int d, int act_dtype, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                int32_t* slot_dst, void* x_perm, float* x_perm_scale, void* ws, size_t ws_bytes,
                hipStream_t stream);
size_t moe_permute_workspace_bytes(int T, int E, int k);

/* Activation quantisation for fp8 weights: per token and per 128 channels,
 * s = fp32(amax / 448) (s = 1 when amax is 0 or the quotient underflows to 0),
 * q = e4m3(fp32(x / s)) with IEEE division, nearest-even rounding, saturation at +-448 and the
 * sign kept (negative values that round to zero give 0x80).
 *   x [T][d] bf16 -> xq [T][d] e4m3, xs [T][d/128] fp32. */
int moe_quant_act(const void* x, int T, int d, uint8_t* xq, float* xs, hipStream_t stream);

/* MXFP8 activation quantisation (MOE_DTYPE_MXFP4_A8): per token and per 32 channels, the shared
 * exponent E is the smallest integer with amax <= 448 * 2^E, clamped to [-127, 127] (amax = 0: E = 0);
 * xe = E + 127 (the E8M0 code), xq = e4m3(x * 2^-E) with nearest-even rounding and the sign kept.
 * (GC-MoE, summary: FP4 grouped GEMMs as block-scaled matrix multiplies.)
 *   x [T][d] bf16 -> xq [T][d] e4m3, xe [T][d/32] bytes.  d % 128 == 0. */
int moe_quant_act_mx(const void* x, int T, int d, uint8_t* xq, uint8_t* xe, hipStream_t stream);

/* Grouped expert FFN on expert-contiguous rows: for every expert e with counts[e] > 0, rows
 * [offsets[e], offsets[e]+counts[e]) of x_perm go through (SiLU(X Wg^T) * (X Wu^T)) Wd^T; the result
 * lands in the same rows of y_perm ([rows][d] bf16, rows = offsets[E]).  bf16 weights: x_perm is
 * bf16 and x_perm_scale NULL (also for mxfp4 weights; MOE_DTYPE_MXFP4_A8 quantises those bf16 rows
 * to MXFP8 itself).  fp8 weights: x_perm is e4m3 with x_perm_scale [rows][d/128]; the
 * SwiGLU output is requantised to e4m3 per row and 128 channels before the down GEMM.  Tile
 * shapes are chosen on the device from counts (p->config may force one family).  The shared expert
 * fields of p and w are ignored here.
 *   ws: moe_grouped_ffn_workspace_bytes(p) bytes (rows = T*k of p).  For bf16 weights it includes
 *   64 MiB of partial-sum slots for the GEMMs' last-round split in K. */
int moe_grouped_ffn(const moe_problem* p, const void* x_perm, const float* x_perm_scale,
                    const int32_t* counts, const int32_t* offsets, const moe_weights* w,
                    void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_grouped_ffn_workspace_bytes(const moe_problem* p);

/* MXFP4 weight layout for the library (load time): src holds a row-major matrix of rows x cols
 * E2M1 elements ([rows][cols/2] bytes, element 2j in the low nibble of byte j; stacked experts
 * [E][N][K] are rows = E*N); dst (same size, not overlapping src) receives the tiled layout the
 * expert GEMMs read: per 16-row block and 128-element chunk of a row, 1 KB ordered
 * [g 0..3][row 0..15][16 bytes = elements 32 g .. 32 g + 31 of the chunk], blocks in row-block
 * then chunk order.  rows % 16 == 0 and cols % 128 == 0, else MOE_ERR_UNSUPPORTED; NULL or
 * misaligned (16 bytes) pointers give MOE_ERR_INVALID_ARG.  (GC-MoE, summary: FP4 grouped GEMM;
 * the layout is this library's, so that each wavefront load reads 1 KB contiguously.) */
int moe_mxfp4_tile(const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t stream);

/* fp8 (E4M3) weight layout for the library (load time), as moe_mxfp4_tile with one byte per
 * element: per 16-row block and 128-element chunk, 2 KB ordered [h 0..1][g 0..3][row 0..15]
 * [16 bytes = elements 32 g + 16 h .. + 15 of the chunk].  Same argument rules. */
int moe_fp8_tile(const void* src, void* dst, int64_t rows, int64_t cols, hipStream_t stream);

/* Combine: out[t] = bf16( sum_{j<k} topk_w[t][j] * y_perm[slot_dst[t*k+j]] (+ shared_y[t]) ),
 * the sum in fp32 in increasing j, the shared row (if not NULL) added last.
 *   y_perm [T*k][d] bf16, shared_y [T][d] bf16 or NULL, out [T][d] bf16. */
int moe_combine(const void* y_perm, const int32_t* slot_dst, const float* topk_w, int T, int k,
                int d, const void* shared_y, void* out, hipStream_t stream);

/* The whole layer: route -> permute -> (fp8: quantise activations) -> grouped gate/up + SwiGLU ->
 * grouped down (+ shared expert) -> combine.  The token gather is fused into the gate/up GEMM's
 * activation loads.  For a single bf16 token without a shared expert (T = 1, d <= 8192, config
 * not forcing MFMA tiles) routing, permutation and selection run inside the gate/up kernel: same
 * results and routing outputs, one launch fewer.
 *   logits [T][E] fp32, x [T][d] bf16, out [T][d] bf16.  keep: optional routing outputs.
 *   ws: moe_layer_workspace_bytes(p) bytes (bf16 weights: including 64 MiB of split-K slots). */
int moe_layer(const moe_problem* p, const float* logits, const void* x, const moe_weights* w,
              void* out, const moe_routing* keep, void* ws, size_t ws_bytes, hipStream_t stream);
size_t moe_layer_workspace_bytes(const moe_problem* p);

/* moe_layer with phase timing: records events[0] before the first launch and events[i] after
 * phase i, for the phases route (1), permute (2), activation quantisation (3, empty for bf16),
 * tile selection (4), gate/up GEMM + SwiGLU (5), down GEMM (6) and combine (7).  (In the
 * single-token case of moe_layer phases 1-4 are empty and phase 5 includes them.)  The caller creates
 * the MOE_TRACE_EVENTS events (hipEventCreate) and reads them after the stream has passed them.
 * NULL entries are skipped (each recorded timing event adds a few microseconds of GPU time, so
 * a caller may record only the boundaries it needs).  Same results as moe_layer; num_events must
 * be MOE_TRACE_EVENTS.  Meant for profiling tools
 * ("where the time goes": the pages attribute decode time to dispatch and weight traffic). */
#define MOE_TRACE_EVENTS 8
int moe_layer_traced(const moe_problem* p, const float* logits, const void* x,
                     const moe_weights* w, void* out, const moe_routing* keep, void* ws,
                     size_t ws_bytes, hipEvent_t* events, int num_events, hipStream_t stream);

/* moe_layer without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  The workspace
 * is a static device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU the
 * library runs on, held until the process ends; the caller still passes inputs and outputs.
 * Results are moe_layer's, bit for bit (same kernels).
 *   - MOE_ERR_WORKSPACE if moe_layer_workspace_bytes(p) exceeds MOE_NOALLOC_SCRATCH_BYTES (bf16
 *     DeepSeek-V3-shaped decode fits up to T = 256; Mixtral- or Kimi-shaped prefill does not).
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's contents (the
 *     layer clears what it needs at zero itself): calls that overlap on one GPU -- several
 *     streams or host threads -- race and give wrong results.  Serialise them.
 *   - The first call on a device looks up the array's address there (hipGetSymbolAddress, with that
 *     device current) and keeps it; MOE_ERR_HIP if the lookup fails.  No hipMalloc, hipFree or
 *     other allocation, no synchronisation. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int moe_layer_noalloc(const moe_problem* p, const float* logits, const void* x,
                      const moe_weights* w, void* out, const moe_routing* keep,
                      hipStream_t stream);

/* Static name of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
