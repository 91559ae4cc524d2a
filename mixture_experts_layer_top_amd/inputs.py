"""Seeded synthetic inputs for the fused MoE layer (router logits, activations, expert weights).

This module holds no arithmetic of the layer itself: it only draws inputs. Both the HIP path
(tests, bench) and the CPU oracle (tests) take their inputs from here, and nothing else is shared
between them.

Workloads (the pages measure on models and serving traces that are not available here; these
synthetic draws stand in for them, with the models' layer shapes):
  * "Decoding the Skew: Distribution-Aware MoE Inference with Adaptive Kernel Dispatch",
    Abstract: routing skew is generated with Dirichlet-distributed expert probabilities.  Each
    routing draw takes one p ~ Dirichlet(alpha * 1_E) per layer, and every token's logits are
    log p_e + Gumbel(0, 1), so the top-k of a token samples experts without replacement from p.
  * Near-uniform routing uses fp32 logits ~ N(0, 1).
  * Activations are bf16 ~ N(0, 1): numpy float32 normal draws, rounded to nearest-even bf16.
  * bf16 expert weights are N(0, 0.02)-like.  They are drawn from an integer counter-based hash,
    so that any single expert can be regenerated alone, on the CPU or on a GPU, with identical bits.
    Each value is an Irwin-Hall sum of four 8-bit uniforms (a bounded approximation of a normal
    draw), scaled to std 0.02 with one fp32 multiply and rounded to nearest-even bf16.  Every step
    is exact integer work or a single correctly rounded IEEE operation, so torch on either device
    produces the same bytes.
  * fp8 expert weights are OCP E4M3FN codes with one fp32 scale per 128x128 block.  The codes are
    drawn field by field (sign, exponent field from a table of binade probabilities of a
    half-normal with std 110 truncated at 448, uniform mantissa), so no rounding encoder is
    involved.  Block scales are uniform in [2^-13, 2^-12) with a full random 23-bit mantissa.

Seeds: numpy draws use SeedSequence(entropy=config index, spawn_key=(tag, ...)).  Hash streams use
a 32-bit key folded from (config index, tag, expert).  Python's hash() is never used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

# stream tags
TAG_LOGITS = 1
TAG_DIRICHLET = 2
TAG_X = 3
TAG_W_GATE = 4
TAG_W_UP = 5
TAG_W_DOWN = 6
TAG_SH_GATE = 7
TAG_SH_UP = 8
TAG_SH_DOWN = 9
TAG_SCALE = 16  # added to the weight tag

WDT_BF16 = "bf16"
WDT_FP8 = "fp8"
WDT_MXFP4 = "mxfp4"


@dataclass(frozen=True)
class Problem:
    """Shape and distribution of one MoE-layer workload."""

    name: str
    cfg_index: int
    T: int
    d: int
    f: int
    E: int
    k: int
    routing: str = "normal"  # "normal" (logits ~ N(0,1)) or "dirichlet" (log p + Gumbel)
    alpha: float = 1.0
    wdtype: str = WDT_BF16
    shared: bool = False
    shared_f: int = 0
    w_sigma: float = 0.02
    act_mx8: bool = False  # mxfp4 weights: the layer quantises activations to MXFP8 (per 32)

    def with_T(self, T: int) -> "Problem":
        return replace(self, T=T)


# The five workloads of this layer.  Index = seed entropy.
TINY = Problem("tiny", 0, T=64, d=256, f=512, E=8, k=2)
MIXTRAL = Problem("mixtral_prefill", 1, T=4096, d=4096, f=14336, E=8, k=2)
DSV3_TS = (1, 16, 64, 256)
DSV3_ALPHAS = (0.1, 1.0, 10.0)
DSV3 = Problem("dsv3_decode", 2, T=1, d=7168, f=2048, E=256, k=8, routing="dirichlet", alpha=1.0)
KIMI = Problem("kimi_prefill", 3, T=8192, d=7168, f=2048, E=384, k=8, routing="dirichlet", alpha=0.3)
FP8_TS = (32, 128)
FP8 = Problem("fp8_dsv3_decode", 4, T=32, d=7168, f=2048, E=256, k=8, routing="dirichlet",
              alpha=1.0, wdtype=WDT_FP8, shared=True, shared_f=2048)

# DeepSeek-V3-shaped decode with MXFP4 routed experts (bf16 activations); no shared expert
MXFP4 = Problem("mxfp4_dsv3_decode", 5, T=64, d=7168, f=2048, E=256, k=8, routing="dirichlet",
                alpha=1.0, wdtype=WDT_MXFP4)

# the same layer (weights and routing draws) with MXFP8 activations on the scaled f8f6f4 MFMA
MXFP4_A8 = replace(MXFP4, name="mxfp4a8_dsv3_decode", act_mx8=True)

CONFIGS = {p.name: p for p in (TINY, MIXTRAL, DSV3, KIMI, FP8, MXFP4, MXFP4_A8)}


def dsv3_point(T: int, alpha: float) -> Problem:
    return replace(DSV3, T=T, alpha=alpha, name=f"dsv3_decode_T{T}_a{alpha:g}")


def fp8_point(T: int) -> Problem:
    return replace(FP8, T=T, name=f"fp8_dsv3_decode_T{T}")


def _alpha_key(alpha: float) -> int:
    return int(round(alpha * 1000))


def _seedseq(p: Problem, tag: int, *extra: int) -> np.random.SeedSequence:
    return np.random.SeedSequence(entropy=p.cfg_index, spawn_key=(tag,) + tuple(int(v) for v in extra))


# ---------------------------------------------------------------------------------------------
# numpy draws: logits and activations
# ---------------------------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; returns the uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def gen_logits(p: Problem) -> np.ndarray:
    """Router logits [T, E] float32 (row-major)."""
    if p.routing == "normal":
        rng = np.random.Generator(np.random.PCG64(_seedseq(p, TAG_LOGITS, p.T)))
        return rng.standard_normal((p.T, p.E), dtype=np.float32)
    if p.routing == "dirichlet":
        rng_p = np.random.Generator(np.random.PCG64(_seedseq(p, TAG_DIRICHLET, p.T, _alpha_key(p.alpha))))
        prob = rng_p.dirichlet(np.full(p.E, p.alpha, dtype=np.float64))
        prob = np.maximum(prob, 1e-38)
        rng_g = np.random.Generator(np.random.PCG64(_seedseq(p, TAG_LOGITS, p.T, _alpha_key(p.alpha))))
        g = rng_g.gumbel(0.0, 1.0, size=(p.T, p.E))
        return (np.log(prob)[None, :] + g).astype(np.float32)
    raise ValueError(f"unknown routing {p.routing!r}")


def gen_dirichlet_p(p: Problem) -> np.ndarray:
    """The per-layer expert probabilities behind a Dirichlet routing draw (for statistics)."""
    rng_p = np.random.Generator(np.random.PCG64(_seedseq(p, TAG_DIRICHLET, p.T, _alpha_key(p.alpha))))
    prob = rng_p.dirichlet(np.full(p.E, p.alpha, dtype=np.float64))
    return np.maximum(prob, 1e-38)


# ---------------------------------------------------------------------------------------------
# routing skew as "effective experts"
#
# "Decoding the Skew ..." (Abstract) characterises routing by its Effective Experts and models it
# with Dirichlet draws.  For p ~ Dirichlet(alpha * 1_E) the expected entropy has a closed form,
#     E[-sum_e p_e ln p_e] = psi(E alpha + 1) - psi(alpha + 1)        (psi: digamma),
# and exp of it is the effective expert count of a typical draw; it rises monotonically from 1
# (alpha -> 0) to E (alpha -> infinity), so a target count fixes alpha (bisection in log alpha).
# ---------------------------------------------------------------------------------------------

def expected_entropy(E: int, alpha: float) -> float:
    """Expected entropy (nats) of p ~ Dirichlet(alpha * 1_E)."""
    from scipy.special import digamma
    return float(digamma(E * alpha + 1.0) - digamma(alpha + 1.0))


def expected_eeff(E: int, alpha: float) -> float:
    """exp of the expected entropy: the effective expert count of a typical Dirichlet draw."""
    return math.exp(expected_entropy(E, alpha))


def alpha_for_eeff(E: int, target: float, lo: float = 1e-6, hi: float = 1e6) -> float:
    """The Dirichlet concentration whose draws have `target` effective experts (1 < target < E)."""
    if not 1.0 < target < E:
        raise ValueError(f"effective experts must lie in (1, {E}), got {target}")
    h = math.log(target)
    a, b = math.log(lo), math.log(hi)
    for _ in range(200):
        m = 0.5 * (a + b)
        if expected_entropy(E, math.exp(m)) < h:
            a = m
        else:
            b = m
    return math.exp(0.5 * (a + b))


def effective_experts(counts: np.ndarray) -> float:
    """Effective experts of a routing histogram: exp(-sum q ln q), q = counts / sum(counts)."""
    c = np.asarray(counts, dtype=np.float64)
    q = c[c > 0] / c.sum()
    return float(math.exp(-(q * np.log(q)).sum()))


def gen_x(p: Problem) -> np.ndarray:
    """Activations [T, d] as bf16 bit patterns (uint16)."""
    rng = np.random.Generator(np.random.PCG64(_seedseq(p, TAG_X, p.T)))
    return f32_to_bf16_bits(rng.standard_normal((p.T, p.d), dtype=np.float32))


# ---------------------------------------------------------------------------------------------
# counter-based hash streams (torch, any device)
# ---------------------------------------------------------------------------------------------
_M32 = 0xFFFFFFFF


def _fmix32_int(h: int) -> int:
    """MurmurHash3's 32-bit finaliser (Appleby), on a Python int."""
    h &= _M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & _M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & _M32
    h ^= h >> 16
    return h


def stream_key(cfg_index: int, tag: int, expert: int) -> tuple[int, int]:
    h = 0x6A09E667
    for v in (cfg_index, tag, expert):
        h = _fmix32_int(h ^ _fmix32_int(v + 0x9E3779B9))
    return h, _fmix32_int(h ^ 0xBB67AE85)


def _mul32(x, c: int):
    """(x * c) mod 2^32 for an int64 tensor x in [0, 2^32) and a constant c < 2^32, with no
    intermediate above 2^49 (so no signed overflow on any device)."""
    return ((x & 0xFFFF) * c + (((x >> 16) * (c & 0xFFFF)) << 16)) & _M32


def _fmix32(h):
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def hash_stream(key: tuple[int, int], start: int, n: int, device):
    """32-bit hashes of counters start..start+n-1 under `key`, as an int64 torch tensor."""
    import torch

    if start + n > (1 << 32):
        raise ValueError("counter range exceeds 2^32")
    i = torch.arange(start, start + n, dtype=torch.int64, device=device)
    return _fmix32(_fmix32(i ^ key[0]) ^ key[1])


_IH4_STD = math.sqrt(4.0 * (256.0 ** 2 - 1.0) / 12.0)


def _bf16_bits_from_f32(v):
    import torch

    b = v.view(torch.int32).to(torch.int64) & _M32
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    r = r & 0xFFFF
    r = r - ((r >> 15) << 16)  # to the signed int16 range
    return r.to(torch.int16)


def hashed_normal_bf16(key: tuple[int, int], n: int, sigma: float, device, start: int = 0):
    """n bf16 values (int16 bit patterns) of an Irwin-Hall(4) approximation of N(0, sigma^2)."""
    import torch

    h = hash_stream(key, start, n, device)
    s = (h & 255) + ((h >> 8) & 255) + ((h >> 16) & 255) + (h >> 24) - 510
    c = torch.tensor(sigma / _IH4_STD, dtype=torch.float32, device=device)
    v = s.to(torch.float32) * c
    return _bf16_bits_from_f32(v)


_FP8_SIGMA_Q = 110.0


def _fp8_exponent_thresholds() -> list[int]:
    """Cumulative 24-bit thresholds for the E4M3 exponent field of a half-normal(std 110) truncated
    at 448.  Field 0 covers [0, 2^-6); field f >= 1 covers [2^(f-7), 2^(f-6)), field 15 up to 448."""
    def cdf(v: float) -> float:
        return math.erf(v / (_FP8_SIGMA_Q * math.sqrt(2.0)))

    total = cdf(448.0)
    edges = [0.0] + [2.0 ** (f - 7) for f in range(1, 16)] + [448.0]
    cum = 0.0
    th = []
    for f in range(15):  # thresholds between fields f and f+1
        cum += (cdf(edges[f + 1]) - cdf(edges[f])) / total
        th.append(min(int(round(cum * (1 << 24))), (1 << 24) - 1))
    return th


def hashed_e4m3_codes(key: tuple[int, int], n: int, device, start: int = 0):
    """n OCP E4M3FN codes (uint8), drawn field by field; never the NaN code."""
    import torch

    h = hash_stream(key, start, n, device)
    sign = h >> 31
    mant = (h >> 24) & 7
    u = h & 0xFFFFFF
    th = torch.tensor(_fp8_exponent_thresholds(), dtype=torch.int64, device=device)
    expf = torch.bucketize(u, th, right=True)
    mant = torch.where((expf == 15) & (mant == 7), torch.full_like(mant, 6), mant)
    code = (sign << 7) | (expf << 3) | mant
    return code.to(torch.uint8)


# E2M1 magnitude codes 0..7 stand for 0, 0.5, 1, 1.5, 2, 3, 4, 6; a half-normal of std 2 (in those
# units) split at the midpoints between them gives each code's probability.
_E2M1_SIGMA = 2.0
_E2M1_EDGES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _e2m1_thresholds() -> list[int]:
    """Cumulative 15-bit thresholds between the E2M1 magnitude codes of a half-normal(std 2)."""
    return [min(int(round(math.erf(v / (_E2M1_SIGMA * math.sqrt(2.0))) * (1 << 15))), (1 << 15) - 1)
            for v in _E2M1_EDGES]


def hashed_e2m1_bytes(key: tuple[int, int], nbytes: int, device, start: int = 0):
    """nbytes bytes of packed E2M1 codes (two per byte, low nibble first), each code drawn field by
    field from 16 hash bits: a uniform sign and a magnitude code from a 15-bit uniform."""
    import torch

    h = hash_stream(key, start, nbytes, device)
    th = torch.tensor(_e2m1_thresholds(), dtype=torch.int64, device=device)
    nib = []
    for half in (h & 0xFFFF, h >> 16):
        mag = torch.bucketize(half & 0x7FFF, th, right=True)
        nib.append(((half >> 15) << 3) | mag)
    return (nib[0] | (nib[1] << 4)).to(torch.uint8)


def hashed_e8m0_scales(key: tuple[int, int], n: int, device):
    """n E8M0 scale codes, uniform over 120..124 (2^-7 ... 2^-3)."""
    import torch

    h = hash_stream(key, 0, n, device)
    return (120 + (h >> 8) % 5).to(torch.uint8)


def hashed_block_scales(key: tuple[int, int], n: int, device):
    """n fp32 block scales, uniform in [2^-13, 2^-12) with a random 23-bit mantissa (exact)."""
    import torch

    h = hash_stream(key, 0, n, device)
    m = (1 << 23) + (h >> 9)
    return m.to(torch.float32) * (2.0 ** -36)


# ---------------------------------------------------------------------------------------------
# expert weights
# ---------------------------------------------------------------------------------------------
# Storage (row-major, the contraction dim contiguous):
#   gate, up : [E, f, d]  (math shape d x f, stored transposed)
#   down     : [E, d, f]  (math shape f x d, stored transposed)
#   fp8 block scales: gate/up [E, f/128, d/128], down [E, d/128, f/128]
#   mxfp4: packed E2M1 gate/up [E, f, d/2], down [E, d, f/2] (low nibble = even column) and E8M0
#          scales gate/up [E, f, d/32], down [E, d, f/32], one per 32 along the contraction dim
WEIGHT_TAGS = {"gate": TAG_W_GATE, "up": TAG_W_UP, "down": TAG_W_DOWN,
               "sh_gate": TAG_SH_GATE, "sh_up": TAG_SH_UP, "sh_down": TAG_SH_DOWN}


def weight_shape(p: Problem, which: str) -> tuple[int, int]:
    if which in ("gate", "up"):
        return (p.f, p.d)
    if which == "down":
        return (p.d, p.f)
    if which in ("sh_gate", "sh_up"):
        return (p.shared_f, p.d)
    if which == "sh_down":
        return (p.d, p.shared_f)
    raise ValueError(which)


def gen_expert_weight(p: Problem, which: str, e: int, device="cpu"):
    """One expert's stored weight matrix: int16 bf16 bits, uint8 e4m3 codes for fp8, or packed
    uint8 E2M1 pairs [rows, cols/2] for mxfp4."""
    rows, cols = weight_shape(p, which)
    key = stream_key(p.cfg_index, WEIGHT_TAGS[which], e)
    if p.wdtype == WDT_BF16:
        return hashed_normal_bf16(key, rows * cols, p.w_sigma, device).view(rows, cols)
    if p.wdtype == WDT_MXFP4:
        return hashed_e2m1_bytes(key, rows * cols // 2, device).view(rows, cols // 2)
    return hashed_e4m3_codes(key, rows * cols, device).view(rows, cols)


def gen_expert_scales(p: Problem, which: str, e: int, device="cpu"):
    """One expert's scales: fp32 per 128x128 block (fp8), or uint8 E8M0 per 32 along a row
    [rows, cols/32] (mxfp4)."""
    rows, cols = weight_shape(p, which)
    key = stream_key(p.cfg_index, WEIGHT_TAGS[which] + TAG_SCALE, e)
    if p.wdtype == WDT_MXFP4:
        return hashed_e8m0_scales(key, rows * (cols // 32), device).view(rows, cols // 32)
    return hashed_block_scales(key, (rows // 128) * (cols // 128), device).view(rows // 128, cols // 128)


def gen_weights(p: Problem, device="cpu") -> dict:
    """All expert weights as stacked torch tensors on `device` (generated one expert at a time)."""
    import torch

    out = {}
    wdt = torch.int16 if p.wdtype == WDT_BF16 else torch.uint8
    if p.wdtype == WDT_MXFP4 and p.shared:
        raise ValueError("mxfp4 weights: no shared expert")
    for which in ("gate", "up", "down"):
        rows, cols = weight_shape(p, which)
        wcols = cols // 2 if p.wdtype == WDT_MXFP4 else cols
        t = torch.empty((p.E, rows, wcols), dtype=wdt, device=device)
        for e in range(p.E):
            t[e] = gen_expert_weight(p, which, e, device)
        out[which] = t
        if p.wdtype == WDT_FP8:
            s = torch.empty((p.E, rows // 128, cols // 128), dtype=torch.float32, device=device)
            for e in range(p.E):
                s[e] = gen_expert_scales(p, which, e, device)
            out["s_" + which] = s
        elif p.wdtype == WDT_MXFP4:
            s = torch.empty((p.E, rows, cols // 32), dtype=torch.uint8, device=device)
            for e in range(p.E):
                s[e] = gen_expert_scales(p, which, e, device)
            out["s_" + which] = s
    if p.shared:
        for which in ("sh_gate", "sh_up", "sh_down"):
            out[which] = gen_expert_weight(p, which, 0, device)
            if p.wdtype == WDT_FP8:
                out["s_" + which] = gen_expert_scales(p, which, 0, device)
    return out
