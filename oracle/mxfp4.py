"""MXFP4 weights (OCP microscaling: FP4 E2M1 elements, one E8M0 scale per 32), written from the
format definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The GC-MoE page (summary) names FP4 grouped GEMMs with block-scaled MMA and in-register FP4
decoding but does not fix the 4-bit format; this uses the OCP Microscaling Formats (MX) v1.0
MXFP4 format, the one gfx950's scaled conversions and MFMAs take:
  element E2M1, bit layout S.EE.M, exponent bias 1, no infinities or NaN:
    E = 0     : subnormal, value (-1)^S * M * 2^-1            (0 or 0.5)
    E = 1..3  : normal,    value (-1)^S * (1 + M/2) * 2^(E-1)  (1 ... 6)
  scale E8M0, an 8-bit biased exponent: value 2^(X - 127) for X = 0..254; X = 255 is NaN.
  A block is 32 consecutive elements along the contraction dimension sharing one scale.
Storage (the library's layout): row-major [R, C/2] bytes, element 2j in the low nibble of byte j
and element 2j+1 in the high nibble; scales [R, C/32], one byte per block of 32 along a row.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E2M1_MAX = 6.0
E8M0_NAN = 255


def _e2m1_formula(c) -> np.ndarray:
    s = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    sub = m * 0.5
    nor = np.ldexp(1.0 + m / 2.0, e - 1)
    mag = np.where(e == 0, sub, nor)
    return np.where(s == 1, -mag, mag)


def _e8m0_formula(a) -> np.ndarray:
    v = np.ldexp(1.0, a - 127)
    return np.where(a == E8M0_NAN, np.nan, v)


# every code's value, from the formulas above (a lookup of these tables is the decoder)
_E2M1 = _e2m1_formula(np.arange(16, dtype=np.int64))
_E8M0 = _e8m0_formula(np.arange(256, dtype=np.int64))


def decode_e2m1(codes) -> np.ndarray:
    """4-bit codes (0..15, any integer dtype) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 15)):
        raise ValueError("E2M1 codes are 4-bit")
    return _E2M1[c]


def decode_e8m0(x) -> np.ndarray:
    """8-bit E8M0 scale codes -> float64 (NaN for 255)."""
    return _E8M0[np.asarray(x, dtype=np.uint8)]


def unpack(packed) -> np.ndarray:
    """[R, C/2] bytes -> [R, C] 4-bit codes (low nibble first)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def dequant(packed, scales) -> np.ndarray:
    """MXFP4 matrix: packed [R, C/2] uint8, scales [R, C/32] uint8 -> float64 [R, C]."""
    v = decode_e2m1(unpack(packed))
    s = decode_e8m0(np.asarray(scales, dtype=np.uint8))
    if v.shape[-1] != BLOCK * s.shape[-1] or v.shape[:-1] != s.shape[:-1]:
        raise ValueError(f"scales {s.shape} do not match elements {v.shape}")
    return v * np.repeat(s, BLOCK, axis=-1)
