"""Group quantizers (oracle).

Asymmetric min-max B-bit quantizer. MixKVQ page, "背景知识与关键观察"
(KV-cache quantization principle) defines z = min(X), s = (max - min)/(2^B - 1),
Q(X) = round((X - z)/s), X~ = Q(X)*s + z. The KIVI blog section 2 makes the
rounding round-half-to-even and the origin a float in value units. PN-Mix
page "核心公式" Eq.2 adds clip(., 0, 2^b - 1) and states that a constant group
keeps scale zero and offset equal to the original value.

Readings fixed here (where the pages leave a step open):
* the code is RNE of the EXACT rational (2^B - 1)(x - m)/(M - m), not of a
  division by an already rounded step (the KIVI teaching code divides by a
  float step; on its worked examples both agree);
* scale and offset are stored as IEEE binary16: PN-Mix's GPU path keeps its
  metadata in FP16 (section "本地复现"), and the KIVI blog's storage budget
  (section 7) prices origin and step as FP16 each. The scale is the binary16
  nearest to the exact real (M - m)/(2^B - 1) (ties to even); the offset is
  the binary16 nearest to the group minimum, which is exact for bf16 inputs
  inside the binary16 range. A scale or offset beyond that range is stored as
  infinity (the flush raises a range flag for it);
* a constant group (M == m) stores codes 0, scale +0.0 and offset m;
* a zero scale or offset is stored as +0.0.

1-bit midpoint correction (PN-Mix page "核心公式" Eq.7): s = (M - m)/2,
z = (3m + M)/4 and q = clip(round((x - z)/s), 0, 1). Worked out exactly,
(x - z)/s = 2(x - m)/(M - m) - 1/2, so the code is 1 iff 2(x - m) > M - m; a
value exactly at the midpoint rounds half-to-even to 0.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .numerics import bf16_fraction, f16_to_f64, rn_f16_meta_bits

_SPAN_LIMIT = 48   # int64 path is exact while the group's binade span is <= this


def _decompose(bits: np.ndarray):
    """bf16 bits -> (signed integer significand, exponent) with value = s * 2**e."""
    b = bits.astype(np.int64)
    sign = np.where(b & 0x8000, -1, 1)
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    if np.any(e == 0xFF):
        raise ValueError("non-finite input")
    sig = np.where(e > 0, m + 128, m) * sign
    ex = np.maximum(e, 1) - 134
    return sig, ex


def _exact_ints(bits: np.ndarray):
    """Per-row exact integer representation X = value / 2**e0 (row = group).

    Returns (X, e0) with X int64 when every row spans at most _SPAN_LIMIT
    binades, else a Python-int object array."""
    sig, ex = _decompose(bits)
    nz = sig != 0
    big = np.iinfo(np.int64).max
    e0 = np.where(nz, ex, big).min(axis=1)
    e0 = np.where(e0 == big, 0, e0)
    shift = np.where(nz, ex - e0[:, None], 0)
    if shift.max(initial=0) <= _SPAN_LIMIT:
        return sig << shift, e0
    X = np.empty(sig.shape, dtype=object)
    for idx in np.ndindex(sig.shape):
        X[idx] = int(sig[idx]) << int(shift[idx])
    return X, e0


def _rne_div_vec(num, den):
    q = num // den
    r = num - q * den
    up = (2 * r > den) | ((2 * r == den) & (q % 2 == 1))
    return q + up.astype(q.dtype) if q.dtype != object else q + up


def _min_bits(bits_row, X_row):
    """binary16 offset bits of the row minimum (a bf16 input value)."""
    i = int(np.argmin(X_row))
    return rn_f16_meta_bits(bf16_fraction(int(bits_row[i])))


def quantize_groups(bits: np.ndarray, nbits: int):
    """Quantize each row of ``bits`` (uint16 bf16 patterns, [n_groups, G]).

    Returns (codes uint8 [n_groups, G], scale f16 bits [n_groups],
    offset f16 bits [n_groups]). Exact: codes come from integer arithmetic
    on the exact values; the scale is rounded once from the exact rational."""
    bits = np.atleast_2d(np.asarray(bits, dtype=np.uint16))
    levels = (1 << nbits) - 1
    X, e0 = _exact_ints(bits)
    xmin = X.min(axis=1)
    xmax = X.max(axis=1)
    den = xmax - xmin
    const = den == 0
    safe_den = np.where(const, 1, den)
    num = (X - xmin[:, None]) * levels
    codes = _rne_div_vec(num, safe_den[:, None])
    codes = np.where(const[:, None], 0, codes)
    n = bits.shape[0]
    scale = np.zeros(n, dtype=np.uint16)
    offset = np.zeros(n, dtype=np.uint16)
    for g in range(n):
        offset[g] = _min_bits(bits[g], X[g])
        if not const[g]:
            exact = Fraction(int(den[g]), levels) * (Fraction(2) ** int(e0[g]))
            scale[g] = rn_f16_meta_bits(exact)
    return codes.astype(np.uint8), scale, offset


def quantize_groups_midpoint(bits: np.ndarray):
    """1-bit midpoint-corrected quantizer (PN-Mix Eq.7) on each row.

    Returns (codes uint8, scale f16 bits = RN((M-m)/2), offset f16 bits =
    RN((3m+M)/4)); a constant row gives codes 0, scale 0, offset RN(m)."""
    bits = np.atleast_2d(np.asarray(bits, dtype=np.uint16))
    X, e0 = _exact_ints(bits)
    xmin = X.min(axis=1)
    xmax = X.max(axis=1)
    den = xmax - xmin
    const = den == 0
    codes = (2 * (X - xmin[:, None]) > den[:, None]).astype(np.uint8)
    codes = np.where(const[:, None], 0, codes).astype(np.uint8)
    n = bits.shape[0]
    scale = np.zeros(n, dtype=np.uint16)
    offset = np.zeros(n, dtype=np.uint16)
    for g in range(n):
        if const[g]:
            offset[g] = _min_bits(bits[g], X[g])
            continue
        unit = Fraction(2) ** int(e0[g])
        scale[g] = rn_f16_meta_bits(Fraction(int(den[g]), 2) * unit)
        offset[g] = rn_f16_meta_bits(Fraction(3 * int(xmin[g]) + int(xmax[g]), 4) * unit)
    return codes, scale, offset


def dequantize(codes, scale_bits, offset_bits) -> np.ndarray:
    """x^ = offset + scale * code, in float64 (exact for these formats).

    ``scale_bits``/``offset_bits`` (binary16 patterns) broadcast against
    ``codes``."""
    return f16_to_f64(offset_bits) + f16_to_f64(scale_bits) * np.asarray(codes, dtype=np.float64)


def quantize_group_reference(values, nbits: int):
    """Single-group quantizer on exact rationals, restated directly from the
    min-max definition (used to cross-check ``quantize_groups``)."""
    vals = [Fraction(v) for v in values]
    m, M = min(vals), max(vals)
    levels = (1 << nbits) - 1
    if M == m:
        return [0] * len(vals), Fraction(0), m
    codes = []
    for v in vals:
        t = levels * (v - m) / (M - m)
        lo = t.numerator // t.denominator
        frac = t - lo
        c = lo + (1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1) else 0)
        codes.append(min(max(c, 0), levels))
    return codes, (M - m) / levels, m


def bf16_values(bits) -> list:
    """Exact Fractions of bf16 bit patterns."""
    return [bf16_fraction(int(b)) for b in np.asarray(bits).ravel()]
