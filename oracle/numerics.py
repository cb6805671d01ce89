"""Exact number formats used by the oracle.

Everything here is exact: bf16/f16 bit patterns are decoded to Fractions or to
float64 (both formats embed exactly in float64), and rounding a real number to
bf16/f16 is done on an exact rational with round-half-to-even, the rounding
the KIVI blog fixes for codes ("2-bit 量化保存的原点不是整数 zero point", the
RNE in the min-max contract) and the usual IEEE rounding for stored floats.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# (significand bits incl. the implicit one, minimum normal exponent, bias)
_BF16 = (8, -126, 127, 8)   # (p, emin, bias, exponent field width)
_F16 = (11, -14, 15, 5)


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16 array) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits) -> np.ndarray:
    """Decode IEEE binary16 bit patterns (uint16 array) to float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of one bf16 bit pattern (must be finite)."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite bf16")
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(1, 1 << 126)
    val = Fraction(128 + m, 128)
    ex = e - 127
    return sign * (val * (1 << ex) if ex >= 0 else val / (1 << -ex))


def rne_div(num: int, den: int) -> int:
    """round-half-to-even of num/den for integers num >= 0, den > 0."""
    q, r = divmod(num, den)
    twice = 2 * r
    if twice > den or (twice == den and q % 2 == 1):
        q += 1
    return q


def _round_to_format(x: Fraction, fmt, overflow: str = "raise") -> int:
    p, emin, bias, ew = fmt
    if x == 0:
        return 0
    sign = 0
    if x < 0:
        sign = 1
        x = -x
    n, d = x.numerator, x.denominator
    e = n.bit_length() - d.bit_length()
    # make 2^e <= x < 2^(e+1)
    if (n << max(0, -e)) < (d << max(0, e)):
        e -= 1
    e = max(e, emin)
    shift = e - p + 1                     # quantum = 2^shift
    if shift >= 0:
        m = rne_div(n, d << shift)
    else:
        m = rne_div(n << -shift, d)
    if m == (1 << p):                     # rounded up into the next binade
        m >>= 1
        e += 1
    if m < (1 << (p - 1)):                # subnormal (only possible at e == emin)
        exp_field = 0
        mant = m
    else:
        exp_field = e + bias
        mant = m - (1 << (p - 1))
    if exp_field >= (1 << ew) - 1:
        if overflow == "inf":             # IEEE round-to-nearest overflow: +-infinity
            return (sign << (ew + p - 1)) | (((1 << ew) - 1) << (p - 1))
        raise OverflowError("value out of range of the target format")
    return (sign << (ew + p - 1)) | (exp_field << (p - 1)) | mant


def rn_bf16_bits(x: Fraction) -> int:
    """Bit pattern of the bf16 nearest to the exact rational x (ties to even).

    Zero is returned as +0.0."""
    return _round_to_format(Fraction(x), _BF16)


def rn_f16_bits(x: Fraction) -> int:
    """Bit pattern of the IEEE binary16 nearest to x (ties to even)."""
    return _round_to_format(Fraction(x), _F16)


def rn_f16_meta_bits(x: Fraction) -> int:
    """binary16 nearest to x (ties to even) as stored for a quantization scale
    or offset: a value beyond the binary16 range becomes +-infinity (the
    flush reports it), a result that rounds to zero is stored as +0.0."""
    b = _round_to_format(Fraction(x), _F16, overflow="inf")
    return 0 if (b & 0x7FFF) == 0 else b


def f16_fraction(bits: int) -> Fraction:
    """Exact value of one finite binary16 bit pattern."""
    bits = int(bits) & 0xFFFF
    if (bits & 0x7C00) == 0x7C00:
        raise ValueError("non-finite f16")
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    val = Fraction(1024 + m, 1024)
    ex = e - 15
    return sign * (val * (1 << ex) if ex >= 0 else val / (1 << -ex))


def rn_f16_sqrt_bits(s: Fraction) -> int:
    """binary16 nearest to sqrt(s) for an exact rational s >= 0 (ties to even).

    Decided exactly: the candidate is compared with the squared midpoints."""
    if s < 0:
        raise ValueError("negative")
    if s == 0:
        return 0
    approx = Fraction(float(s) ** 0.5)
    c = rn_f16_bits(approx)

    def val(b):
        return Fraction(f16_to_f64(np.array([b], dtype=np.uint16))[0])

    # walk to the correctly rounded neighbour: midpoint tests on squares
    for _ in range(4):
        v = val(c)
        up = val(c + 1) if c + 1 < 0x7C00 else None
        dn = val(c - 1) if c > 0 else None
        if up is not None:
            mid = (v + up) / 2
            if s > mid * mid or (s == mid * mid and (c & 1)):
                c += 1
                continue
        if dn is not None:
            mid = (v + dn) / 2
            if s < mid * mid or (s == mid * mid and (c & 1)):
                c -= 1
                continue
        break
    return c
