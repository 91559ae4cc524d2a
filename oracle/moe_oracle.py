"""The fused MoE layer, step by step, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Slow and plain on purpose: one library
primitive per step at most (a matmul, a bincount), no blocking, no fusion, no reordering.

What the pages fix and what they leave open
-------------------------------------------
The pages describe the layer only at the level of its steps: once routing completes the per-expert
volumes are known (Weave, Abstract); the layer runs sparse expert GEMMs whose shapes follow the live
routing histogram (Decoding the Skew, Abstract); under expert parallelism it pays token dispatch,
grouped GEMMs with fused SwiGLU (and, in FP8, requantisation and optional shared experts) and a
combine step (GC-MoE, summary).  They never write the arithmetic down, so this oracle takes the
plainest reading of a top-k softmax-routed SwiGLU MoE layer:

  route    ids[t] = the k experts with the largest logits, ordered by (-logit, expert id), so ties
           go to the lower id and -0.0 equals +0.0;
           w[t, j] = exp(L[t, ids[t, j]] - L[t, ids[t, 0]]) / sum_j' exp(L[t, ids[t, j']] - ...),
           i.e. the softmax renormalised over the selected logits.
  dispatch counts[e] = number of slots s = t*k + j with ids[t, j] = e; offsets = exclusive prefix
           sum (offsets[E] = T*k); slots are placed expert by expert, in increasing s inside an
           expert (a stable counting sort): perm_src[row] = s, slot_dst[s] = row.  No capacity
           limit, no dropped tokens, no padding in the exported layout.
  experts  for every expert with counts[e] > 0, on its rows X_e = x[perm_src[row] // k]:
           G = X_e Wg^T, U = X_e Wu^T (Wg, Wu stored [f, d]), H = SiLU(G) * U with
           SiLU(z) = z * sigmoid(z), Y_e = H Wd^T (Wd stored [d, f]).  No biases, no clamp.
  shared   (optional) one always-active SwiGLU expert on all T tokens, added with weight 1 outside
           the renormalisation.
  combine  out[t] = sum_j w[t, j] * Y[slot_dst[t*k + j]] (+ S[t]).
  fp8      weights are OCP E4M3FN codes with one fp32 scale per 128x128 block and are used as
           code * scale.  Activations are quantised by the layer, per token and per 128 channels:
           s = fp32(amax / 448) (s = 1 when amax = 0), q = e4m3(fp32(x / s)); the experts then see
           q * s.  The oracle runs the experts on these dequantised values in float64 and does not
           requantise H.
  mxfp8    (MXFP4 weights with 8-bit activations) activations are quantised by the layer to OCP
           MXFP8, per token and per 32 channels (oracle/mxfp8.py); the experts see the dequantised
           values, and again H is not requantised.

Every function below follows one of these steps; all arithmetic is float64 unless stated.
"""
from __future__ import annotations

import numpy as np

from . import fp8_e4m3, mxfp4, mxfp8

ACT_BLOCK = 128  # activation quantisation group (channels)
W_BLOCK = 128  # weight scale block edge


# ---------------------------------------------------------------------------------------------
# storage decoding
# ---------------------------------------------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16 / int16) -> exact float32 values."""
    b = np.asarray(bits).view(np.uint16) if np.asarray(bits).dtype == np.int16 else np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def f64_to_bf16_f64(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to an even last bit (returned as
    float64), in one rounding straight from float64.

    bfloat16 has 8 significant bits and float32's exponent range: a value v = m * 2^e with
    0.5 <= |m| < 1 lies on the grid of its quantum 2^(e - 8) while e >= -125 (normal numbers,
    down to 2^-126); below that the grid is the subnormal quantum 2^-133.  A result of magnitude
    2^128 or more is out of range and becomes an infinity of the value's sign."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e, -125) - 8  # exponent of the quantum
    r = np.round(np.ldexp(v, -q))  # scaling by a power of two is exact; numpy rounds half to even
    out = np.ldexp(r, q)
    out = np.where(np.abs(out) >= 2.0 ** 128, np.copysign(np.inf, v), out)
    return np.where(v == 0, v, out)


def dequant_e4m3_blocks(codes, scales) -> np.ndarray:
    """Block-scaled E4M3 weights: codes [R, C] uint8, scales [R/128, C/128] fp32 -> float64."""
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    v = fp8_e4m3.decode(c)
    return v * np.repeat(np.repeat(s, W_BLOCK, axis=0), W_BLOCK, axis=1)


def decode_weight(raw, scales=None) -> np.ndarray:
    """Stored expert weight -> float64: bf16 bits; E4M3 codes with fp32 128x128 block scales; or
    packed MXFP4 (E2M1 pairs) with uint8 E8M0 scales per 32 along a row."""
    a = np.asarray(raw)
    if a.dtype == np.uint8:
        if scales is None:
            raise ValueError("fp8 and mxfp4 weights need scales")
        sc = np.asarray(scales)
        if sc.dtype == np.uint8:
            return mxfp4.dequant(a, sc)
        return dequant_e4m3_blocks(a, sc)
    return bf16_bits_to_f64(a)


# ---------------------------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------------------------

def route(logits, k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Returns ids int32 [T, k] (descending logit, ties to the lower id) and w float64 [T, k]."""
    L = np.asarray(logits, dtype=np.float32).astype(np.float64) + 0.0  # -0.0 -> +0.0
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-L, axis=1, kind="stable")  # equal values keep increasing expert id
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(L, ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel[:, :1])
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


# ---------------------------------------------------------------------------------------------
# dispatch: histogram, prefix sum, stable permutation
# ---------------------------------------------------------------------------------------------

def histogram(ids, E: int):
    """counts[e] = #slots routed to e; offsets = exclusive prefix sum with offsets[E] = T*k."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    return counts, offsets


def permute(ids, E: int):
    """Stable counting sort of the slots s = t*k + j by expert.

    Walks the slots in increasing s; each takes the next free row of its expert's segment.
    Returns perm_src[row] = s and slot_dst[s] = row (both int64, length T*k)."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    _, offsets = histogram(ids, E)
    cursor = offsets[:-1].copy()
    n = flat.size
    perm_src = np.empty(n, dtype=np.int64)
    slot_dst = np.empty(n, dtype=np.int64)
    for s in range(n):
        e = flat[s]
        row = cursor[e]
        cursor[e] += 1
        perm_src[row] = s
        slot_dst[s] = row
    return perm_src, slot_dst


# ---------------------------------------------------------------------------------------------
# experts
# ---------------------------------------------------------------------------------------------

def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, Wg, Wu, Wd):
    """SwiGLU expert on rows X [m, d]: (SiLU(X Wg^T) * (X Wu^T)) Wd^T, with Wg, Wu [f, d], Wd [d, f]."""
    G = X @ Wg.T
    U = X @ Wu.T
    H = silu(G) * U
    return H @ Wd.T


# ---------------------------------------------------------------------------------------------
# fp8 activation quantisation (per token, per 128 channels)
# ---------------------------------------------------------------------------------------------

def quant_act_e4m3(x_bits):
    """x bf16 bits [T, d] -> (codes uint8 [T, d], scales float32 [T, d/128]).

    s = fp32(amax / 448) over each 1x128 group (s = 1 when amax = 0 or the quotient underflows
    to 0), q = e4m3(fp32(x / s)) with the saturating nearest-even encoder.  Float32 division is
    IEEE (correctly rounded) here, as the reading requires of both sides."""
    x = bf16_bits_to_f32(x_bits)
    T, d = x.shape
    if d % ACT_BLOCK:
        raise ValueError("d must be a multiple of 128")
    xb = x.reshape(T, d // ACT_BLOCK, ACT_BLOCK)
    amax = np.abs(xb).max(axis=2)
    s = (amax / np.float32(fp8_e4m3.E4M3_MAX)).astype(np.float32)
    s = np.where((amax == 0) | (s == 0), np.float32(1.0), s).astype(np.float32)
    r = (xb / s[:, :, None]).astype(np.float32)
    q = fp8_e4m3.encode(r.astype(np.float64)).reshape(T, d)
    return q, s


def dequant_act_e4m3(q, s) -> np.ndarray:
    T, d = q.shape
    v = fp8_e4m3.decode(q).reshape(T, d // ACT_BLOCK, ACT_BLOCK)
    return (v * np.asarray(s, dtype=np.float32).astype(np.float64)[:, :, None]).reshape(T, d)


# ---------------------------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------------------------

def _expert_mats(get_weights, e):
    raw = get_weights(e)
    return (decode_weight(raw["gate"], raw.get("s_gate")),
            decode_weight(raw["up"], raw.get("s_up")),
            decode_weight(raw["down"], raw.get("s_down")))


ACTS = ("bf16", "fp8", "mxfp8")


def _act(act_fp8, act):
    """The activation format: act if given, else 'fp8' or 'bf16' from the older act_fp8 flag."""
    a = act if act is not None else ("fp8" if act_fp8 else "bf16")
    if a not in ACTS:
        raise ValueError(f"activation format {a!r} not in {ACTS}")
    return a


def layer_input(x_bits, act_fp8: bool = False, act: str | None = None):
    """What the experts see: the bf16 activations, their per-token fp8 quantisation (1x128, fp32
    scales) or their MXFP8 quantisation (1x32, E8M0 scales).  Returns (values, codes, scales)."""
    a = _act(act_fp8, act)
    if a == "fp8":
        q, s = quant_act_e4m3(x_bits)
        return dequant_act_e4m3(q, s), q, s
    if a == "mxfp8":
        q, s = mxfp8.quant_act(x_bits)
        return mxfp8.dequant_rows(q, s), q, s
    return bf16_bits_to_f64(x_bits), None, None


def combine(Y, slot_dst, w, S=None):
    """out[t] = sum_j w[t, j] * Y[slot_dst[t*k + j]] (+ S[t])."""
    T, k = w.shape
    rows = np.asarray(slot_dst, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * Y[rows[:, j]]
    if S is not None:
        out += S
    return out


def moe_layer(logits, x_bits, k: int, get_weights, get_shared=None, act_fp8: bool = False,
              act: str | None = None):
    """The whole layer.

    logits float32 [T, E]; x_bits bf16 bits [T, d]; get_weights(e) -> dict with the stored
    'gate', 'up' ([f, d]) and 'down' ([d, f]) of expert e (bf16 bits, or E4M3 codes plus
    's_gate', 's_up', 's_down' block scales); get_shared() -> the same for the shared expert.
    Returns a dict of every intermediate the boundary exports plus 'out' (float64 [T, d]).
    act: activation format ('bf16', 'fp8', 'mxfp8'; act_fp8=True is 'fp8')."""
    return moe_layers([(logits, x_bits)], k, get_weights, get_shared, act_fp8, act)[0]


def moe_layers(batches, k: int, get_weights, get_shared=None, act_fp8: bool = False,
               act: str | None = None):
    """Several calls of the layer with one set of expert weights (a sweep over batch sizes or
    routing draws of one model layer), each computed exactly as moe_layer defines it; an expert's
    weights are decoded once for all the calls that route rows to it.

    batches: list of (logits float32 [T_i, E], x_bits bf16 bits [T_i, d]).  Returns one result dict
    per call (see moe_layer)."""
    a = _act(act_fp8, act)
    res = []
    for logits, x_bits in batches:
        logits = np.asarray(logits, dtype=np.float32)
        T, E = logits.shape
        ids, w = route(logits, k)
        counts, offsets = histogram(ids, E)
        perm_src, slot_dst = permute(ids, E)
        xin, xq, xs = layer_input(x_bits, act=a)
        r = dict(ids=ids, w=w, counts=counts, offsets=offsets, perm_src=perm_src,
                 slot_dst=slot_dst, y_perm=np.zeros((T * k, xin.shape[1]), dtype=np.float64),
                 xin=xin)
        if a != "bf16":
            r["xq"], r["xs"] = xq, xs
        res.append(r)
    E = res[0]["counts"].size if res else 0
    for e in range(E):
        if all(int(r["counts"][e]) == 0 for r in res):
            continue
        Wg, Wu, Wd = _expert_mats(get_weights, e)
        for r in res:
            c = int(r["counts"][e])
            if c == 0:
                continue
            r0 = int(r["offsets"][e])
            tokens = r["perm_src"][r0:r0 + c] // k
            r["y_perm"][r0:r0 + c] = expert_ffn(r["xin"][tokens], Wg, Wu, Wd)
    sh = None
    if get_shared is not None:
        raw = get_shared()
        sh = (decode_weight(raw["gate"], raw.get("s_gate")), decode_weight(raw["up"], raw.get("s_up")),
              decode_weight(raw["down"], raw.get("s_down")))
    for r in res:
        S = expert_ffn(r["xin"], *sh) if sh is not None else None
        r["out"] = combine(r["y_perm"], r["slot_dst"], r["w"], S)
        if S is not None:
            r["shared_y"] = S
        del r["xin"]
    return res


def moe_tokens(tokens, logits, x_bits, k: int, get_weights, get_shared=None, act_fp8: bool = False,
               act: str | None = None):
    """Output rows for a subset of tokens, computed token by token with no permutation:
    out[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x_t) (+ FFN_shared(x_t)).  Routing, the fp8
    activation quantisation and the experts all act row by row, so this needs only the chosen
    tokens and the experts they route to."""
    tokens = np.asarray(tokens, dtype=np.int64)
    logits = np.asarray(logits, dtype=np.float32)[tokens]
    x_sel = np.asarray(x_bits)[tokens]
    ids, w = route(logits, k)
    xin, _, _ = layer_input(x_sel, act_fp8, act)
    out = np.zeros((tokens.size, xin.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        Wg, Wu, Wd = _expert_mats(get_weights, int(e))
        tt, jj = np.nonzero(ids == e)
        Ye = expert_ffn(xin[tt], Wg, Wu, Wd)
        out[tt] += w[tt, jj][:, None] * Ye
    if get_shared is not None:
        raw = get_shared()
        out += expert_ffn(xin, decode_weight(raw["gate"], raw.get("s_gate")),
                          decode_weight(raw["up"], raw.get("s_up")),
                          decode_weight(raw["down"], raw.get("s_down")))
    return dict(ids=ids, w=w, out=out)


# ---------------------------------------------------------------------------------------------
# a rounding-emulating variant (diagnostic: shows the output tolerance is attainable)
# ---------------------------------------------------------------------------------------------

def quant_rows_e4m3_f64(v):
    """Per-row, per-128 requantisation of float64 values through float32 (used by the emulated
    variant for the fp8 H requantisation)."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    R, C = v32.shape
    b = v32.reshape(R, C // ACT_BLOCK, ACT_BLOCK)
    amax = np.abs(b).max(axis=2)
    s = (amax / np.float32(fp8_e4m3.E4M3_MAX)).astype(np.float32)
    s = np.where((amax == 0) | (s == 0), np.float32(1.0), s).astype(np.float32)
    q = fp8_e4m3.encode((b / s[:, :, None]).astype(np.float32).astype(np.float64))
    return (fp8_e4m3.decode(q) * s.astype(np.float64)[:, :, None]).reshape(R, C)


def moe_layer_emulated(logits, x_bits, k: int, get_weights, get_shared=None, act_fp8: bool = False,
                       act: str | None = None):
    """Same layer with the rounding a GPU implementation may add: float32 GEMM results, H and Y
    rounded to bf16 (H requantised per 1x128 to fp8 for fp8 activations, per 1x32 to MXFP8 for
    MXFP8 activations), output rounded to bf16."""
    a = _act(act_fp8, act)
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids, w = route(logits, k)
    w = w.astype(np.float32).astype(np.float64)
    counts, offsets = histogram(ids, E)
    perm_src, slot_dst = permute(ids, E)
    xin, _, _ = layer_input(x_bits, act=a)

    def ffn(X, Wg, Wu, Wd):
        G = (X @ Wg.T).astype(np.float32).astype(np.float64)
        U = (X @ Wu.T).astype(np.float32).astype(np.float64)
        H = silu(G) * U
        if a == "fp8":
            H = quant_rows_e4m3_f64(H)
        elif a == "mxfp8":
            H = mxfp8.dequant_rows(*mxfp8.quant_rows(H.astype(np.float32).astype(np.float64)))
        else:
            H = f64_to_bf16_f64(H)
        return f64_to_bf16_f64((H @ Wd.T).astype(np.float32).astype(np.float64))

    Y = np.zeros((T * k, xin.shape[1]), dtype=np.float64)
    for e in range(E):
        c = int(counts[e])
        if c == 0:
            continue
        r0 = int(offsets[e])
        Wg, Wu, Wd = _expert_mats(get_weights, e)
        Y[r0:r0 + c] = ffn(xin[perm_src[r0:r0 + c] // k], Wg, Wu, Wd)
    S = None
    if get_shared is not None:
        raw = get_shared()
        S = ffn(xin, decode_weight(raw["gate"], raw.get("s_gate")),
                decode_weight(raw["up"], raw.get("s_up")),
                decode_weight(raw["down"], raw.get("s_down")))
    return f64_to_bf16_f64(combine(Y, slot_dst, w, S))
