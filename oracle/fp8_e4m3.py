"""OCP E4M3FN (8-bit float) codec, written from the format definition.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The GC-MoE page (summary) names FP8 block-scaled grouped GEMMs with requantisation but does not fix
the 8-bit format; this uses the OCP 8-bit floating point specification's E4M3 encoding, which is
the native fp8 of gfx950 MFMA (not the FNUZ variant of gfx942):
  bit layout S.EEEE.MMM, exponent bias 7;
  E = 0        : subnormal, value (-1)^S * (M/8) * 2^-6;
  E = 1..15    : normal, value (-1)^S * (1 + M/8) * 2^(E-7);
  S.1111.111   : NaN (the only non-finite codes); there are no infinities;
  largest finite magnitude S.1111.110 = 1.75 * 2^8 = 448; smallest subnormal 2^-9.

Encoding (the reading used on both sides of the parity check): round to nearest, ties to the code
with an even mantissa, saturate magnitudes above 448 to 448, keep the sign (so negative values that
round to zero give the code 0x80).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def _decode_formula(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for S.1111.111), from the bit layout above."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    sub = np.ldexp(m / 8.0, -6)
    nor = np.ldexp(1.0 + m / 8.0, e - 7)
    mag = np.where(e == 0, sub, nor)
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return val


# every code's value, from the formula (a lookup of this table is the decoder)
_TABLE = _decode_formula(np.arange(256, dtype=np.uint8))


def decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for S.1111.111)."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


# non-negative finite values, codes 0..126, strictly increasing in the code
_POS = _TABLE[:127].copy()


def encode(v) -> np.ndarray:
    """float64 values -> uint8 codes: nearest, ties to even mantissa, saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    a = np.where(np.isnan(v), 0.0, a)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(take_hi, hi, lo)
    code = (sign << 7) | mag
    code = np.where(np.isnan(v), NAN_CODE, code)
    return code.astype(np.uint8)
