"""MXFP8 activations (OCP microscaling: FP8 E4M3 elements, one E8M0 scale per 32), written from the
format definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The GC-MoE page (summary) runs FP4 grouped GEMMs as block-scaled matrix multiplies; on gfx950 the
scaled f8f6f4 matrix instruction takes both operands block-scaled, so the FP4 expert weights (OCP
MXFP4, oracle/mxfp4.py) meet activations in OCP MXFP8: E4M3 elements (oracle/fp8_e4m3.py) sharing
one E8M0 scale 2^(X - 127) per block of 32 consecutive channels.  The pages do not say how the
activations get their scales; the reading here:

  per token and per block of 32 channels, amax = max |x_i|;
  amax = 0: X = 127 (scale 1) and every element encodes its signed zero;
  otherwise the shared exponent E is the smallest integer with amax <= 448 * 2^E (448 = E4M3's
  largest finite value), clamped to E8M0's range [-127, 127], and X = E + 127;
  q_i = E4M3(x_i * 2^-E), nearest with ties to even (saturating at +-448 only when the clamp bites),
  sign kept.
So the block's largest element lands in (224, 448] and no element is clipped.  (The MX format
document's own conversion takes E = floor(log2(amax)) - 8, which puts the largest element in
[256, 512) and clips it to 448 in about one block in seven, by up to 12.5%; with h requantised that
way a rounding-emulating layer already misses the 6e-2 output bound.)
Dequantised: x_i = e4m3(q_i) * 2^E.  The same rule requantises the SwiGLU output h (float32 values)
before the down GEMM on the GPU; the oracle keeps h in float64.
"""
from __future__ import annotations

import numpy as np

from . import fp8_e4m3

BLOCK = 32
ELEM_EMAX = 8          # exponent of E4M3's largest normal binade
SCALE_BIAS = 127


def shared_exponent(amax) -> np.ndarray:
    """E = the smallest integer with amax <= 448 * 2^E, clamped to [-127, 127] (amax > 0); 0 where
    amax == 0.  From the binade of amax: with amax in [2^(E0 + 8), 2^(E0 + 9)), amax * 2^-E0 lies in
    [256, 512), and E = E0 + 1 exactly when that exceeds 448."""
    a = np.asarray(amax, dtype=np.float64)
    pos = a > 0
    _, e = np.frexp(np.where(pos, a, 1.0))  # a = m * 2^e, 0.5 <= m < 1: floor(log2 a) = e - 1
    E0 = e - 1 - ELEM_EMAX
    E = E0 + (np.ldexp(np.where(pos, a, 1.0), -E0) > fp8_e4m3.E4M3_MAX)
    E = np.clip(E, -SCALE_BIAS, SCALE_BIAS)
    return np.where(pos, E, 0).astype(np.int64)


def quant_rows(v):
    """float values [R, C] (exact in float64) -> (E4M3 codes uint8 [R, C], E8M0 scale codes uint8
    [R, C/32]) by the rule above."""
    v = np.asarray(v, dtype=np.float64)
    R, C = v.shape
    if C % BLOCK:
        raise ValueError("the channel count must be a multiple of 32")
    b = v.reshape(R, C // BLOCK, BLOCK)
    E = shared_exponent(np.abs(b).max(axis=2))
    q = fp8_e4m3.encode(np.ldexp(b, -E[:, :, None])).reshape(R, C)
    return q, (E + SCALE_BIAS).astype(np.uint8)


def dequant_rows(q, x) -> np.ndarray:
    """E4M3 codes [R, C] and E8M0 scale codes [R, C/32] -> float64 [R, C]."""
    q = np.asarray(q, dtype=np.uint8)
    R, C = q.shape
    E = np.asarray(x, dtype=np.int64) - SCALE_BIAS
    v = fp8_e4m3.decode(q).reshape(R, C // BLOCK, BLOCK)
    return np.ldexp(v, E[:, :, None]).reshape(R, C)


def quant_act(x_bits):
    """bf16 activation bits [T, d] -> (codes uint8 [T, d], scale codes uint8 [T, d/32])."""
    b = np.asarray(x_bits).view(np.uint16) if np.asarray(x_bits).dtype == np.int16 \
        else np.asarray(x_bits, dtype=np.uint16)
    x = (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return quant_rows(x)
