"""Pins of the oracle's group quantizers against what the pages fix.

* KIVI blog section 3 worked examples (per-channel Key exact, per-token row
  0 of the Key, per-token Value exact, per-channel Value 100/3),
  the low-bits-first packing example (0xE4) and the constant groups;
* MixKVQ appendix error bound |x - x^| <= s/2 (exact grid);
* RNE ties (KIVI blog section 2 contract) on constructed exact ties;
* PN-Mix Eq.7 midpoint levels (3m+M)/4 and (m+3M)/4, error <= (M-m)/4;
* brute force against a direct nearest-level search on small groups.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import layout
from oracle.numerics import bf16_fraction, bf16_to_f64, f16_fraction, f16_to_f64
from oracle.quant import (dequantize, quantize_group_reference, quantize_groups,
                          quantize_groups_midpoint)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def bf(values):
    a = np.asarray(values, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (u >> 16).astype(np.uint16)


def exact_grid(codes, nbits, group_bits):
    vals = [bf16_fraction(int(b)) for b in group_bits]
    m, M = min(vals), max(vals)
    step = (M - m) / ((1 << nbits) - 1)
    return [m + int(c) * step for c in codes], step


def qdq_rows_exact(mat, nbits=2):
    out = []
    for row in mat:
        bits = bf(row)
        codes, _, _ = quantize_groups(bits[None, :], nbits)
        grid, _ = exact_grid(codes[0], nbits, bits)
        out.append([float(v) for v in grid])
    return np.array(out)


@pytest.fixture(scope="module")
def kivi():
    with open(os.path.join(GOLD, "kivi_axes_examples.json")) as f:
        return json.load(f)


def test_key_per_channel_exact_per_token_polluted(kivi):
    K = np.array(kivi["key_matrix"]["K"])
    per_channel = qdq_rows_exact(K.T).T
    per_token = qdq_rows_exact(K)
    assert np.array_equal(per_channel, K)
    assert per_token[0].tolist() == kivi["key_matrix"]["per_token_row0"]


def test_key_attention_decision_flips(kivi):
    K = np.array(kivi["key_matrix"]["K"])
    q = np.array(kivi["key_matrix"]["query"])

    def probs(keys):
        s = keys @ q / math.sqrt(4)
        e = np.exp(s - s.max())
        return e / e.sum()

    p0, pt, pc = probs(K), probs(qdq_rows_exact(K)), probs(qdq_rows_exact(K.T).T)
    assert int(np.argmax(p0)) == kivi["key_matrix"]["argmax_original"]
    assert int(np.argmax(pt)) == kivi["key_matrix"]["argmax_per_token"]
    assert np.array_equal(pc, p0)
    assert np.max(np.abs(p0 - pt)) > kivi["key_matrix"]["min_prob_shift_per_token"]


def test_value_per_token_exact_per_channel_polluted(kivi):
    V = np.array(kivi["value_matrix"]["V"])
    p = np.array(kivi["value_matrix"]["p"])
    out_tok = p @ qdq_rows_exact(V)
    out_ch = p @ qdq_rows_exact(V.T).T
    assert out_tok.tolist() == kivi["value_matrix"]["out_per_token"]
    assert np.allclose(out_ch, 100.0 / 3.0, atol=1e-12, rtol=0)


def test_packing_low_bits_first(kivi):
    pk = kivi["packing"]
    codes, _, _ = quantize_groups(bf(pk["group"])[None, :], 2)
    assert codes[0].tolist() == pk["codes"]
    # a byte of a block holds four codes along the tile axis, low bits first
    X = np.zeros((16, 8, 8), np.uint8)
    for p, c in enumerate(pk["codes"]):
        X[0, p, 0] = c
    blob = layout.pack2_block(X)
    assert blob[0] == pk["packed_byte"] and not blob[1:].any()
    assert np.array_equal(layout.unpack2_block(blob), X)
    # a short row: three codes occupy one byte, the padding is not a code
    X2 = np.zeros((16, 8, 8), np.uint8)
    for p, c in enumerate(pk["short_codes"]):
        X2[0, p, 0] = c
    b2 = layout.pack2_block(X2)
    assert b2[0] == sum(c << (2 * i) for i, c in enumerate(pk["short_codes"]))


def test_constant_groups(kivi):
    for grp in kivi["constant_groups"]["groups"]:
        codes, scale, offset = quantize_groups(bf(grp)[None, :], 2)
        assert not codes.any() and scale[0] == 0
        assert np.array_equal(dequantize(codes[0], scale[0], offset[0]), np.array(grp))
    # negative zero is stored as +0.0
    codes, scale, offset = quantize_groups(np.array([[0x8000, 0x0000, 0x8000, 0x0000]], np.uint16), 2)
    assert offset[0] == 0 and scale[0] == 0


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_error_bound_half_step(nbits):
    rng = np.random.default_rng(nbits)
    x = (rng.standard_normal((400, 128)) * np.exp(rng.uniform(-3, 3, (400, 1)))).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale, offset = quantize_groups(bits, nbits)
    vals = bf16_to_f64(bits)
    m = vals.min(axis=1, keepdims=True)
    M = vals.max(axis=1, keepdims=True)
    step = (M - m) / ((1 << nbits) - 1)
    grid = m + codes * step
    assert np.all(np.abs(vals - grid) <= step / 2 * (1 + 1e-12))
    assert codes.max() <= (1 << nbits) - 1
    # stored (binary16-rounded) scale: bound grows by at most (2^b-1)|s - step|
    s = f16_to_f64(scale)[:, None]
    assert np.all(np.abs(s - step) <= step * 2.0 ** -11)
    rec = dequantize(codes, scale[:, None], offset[:, None])
    assert np.all(np.abs(vals - rec) <= step / 2 + ((1 << nbits) - 1) * np.abs(s - step) + 1e-12)
    # bf16 minima inside the binary16 range are stored exactly
    assert np.array_equal(f16_to_f64(offset)[:, None], m)


def test_rne_ties_go_to_even():
    # m=0, M=3, b=2: step 1; x = 0.5, 1.5, 2.5 are exact ties
    codes, _, _ = quantize_groups(bf([0.0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0, 0.25])[None, :], 2)
    assert codes[0].tolist() == [0, 0, 2, 2, 3, 1, 2, 0]
    # b=4: M-m = 15 -> ties at k + 1/2
    codes4, _, _ = quantize_groups(bf([0.0, 15.0, 0.5, 1.5, 6.5, 7.5, 14.5])[None, :], 4)
    assert codes4[0].tolist() == [0, 15, 0, 2, 6, 8, 14]


def _nearest_level_codes(vals, nbits):
    """Independent characterisation: the level nearest to x, ties to even."""
    m, M = min(vals), max(vals)
    L = (1 << nbits) - 1
    if M == m:
        return [0] * len(vals)
    out = []
    for v in vals:
        best = None
        for c in range(L + 1):
            d = abs(v - (m + c * (M - m) / L))
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        out.append(best[1])
    return out


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_brute_force_small_groups(nbits):
    rng = np.random.default_rng(10 + nbits)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        if trial % 3 == 0:   # small integers: many exact ties
            x = rng.integers(-4, 5, n).astype(np.float32) / 2
        elif trial % 3 == 1:  # wide exponent span -> exercises the big-int path
            x = (rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))).astype(np.float32)
        else:
            x = rng.standard_normal(n).astype(np.float32)
        bits = (x.view(np.uint32) >> 16).astype(np.uint16)
        vals = [bf16_fraction(int(b)) for b in bits]
        codes, scale, offset = quantize_groups(bits[None, :], nbits)
        assert codes[0].tolist() == _nearest_level_codes(vals, nbits)
        ref_codes, ref_step, ref_m = quantize_group_reference(vals, nbits)
        assert codes[0].tolist() == ref_codes
        # metadata: numpy's own double -> binary16 rounding (ties to even,
        # overflow to infinity) of the exact value; the exact value is not a
        # binary16 midpoint to within double precision here
        assert int(offset[0]) == _np_f16_bits(ref_m)
        if ref_step:
            assert int(scale[0]) == _np_f16_bits(ref_step)
            if abs(ref_step) < 65504:
                s = f16_fraction(int(scale[0]))
                # correctly rounded: no binary16 value is closer to the exact step
                e = max(math.floor(math.log2(float(ref_step))), -14)
                assert abs(s - ref_step) <= Fraction(2) ** (e - 10) / 2


def _np_f16_bits(x) -> int:
    with np.errstate(over="ignore"):
        b = int(np.array([float(x)]).astype(np.float16).view(np.uint16)[0])
    return 0 if (b & 0x7FFF) == 0 else b


def test_exhaustive_two_bit_patterns():
    """Every assignment of the levels 0..3 to a 4-element group reconstructs
    exactly when the values sit on an exact grid (step 0.5, origin -1)."""
    for pat in range(256):
        lv = [(pat >> (2 * i)) & 3 for i in range(4)]
        vals = [-1.0 + 0.5 * c for c in lv]
        codes, scale, offset = quantize_groups(bf(vals)[None, :], 2)
        if max(lv) == min(lv):
            assert not codes.any()
            continue
        lo = min(lv)
        span = max(lv) - lo
        grid, _ = exact_grid(codes[0], 2, bf(vals))
        if span == 3:
            assert codes[0].tolist() == [c - lo for c in lv]
            assert [float(g) for g in grid] == vals
        assert codes[0].tolist() == _nearest_level_codes([Fraction(v) for v in vals], 2)


def test_midpoint_one_bit():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    codes, scale, offset = quantize_groups_midpoint(bits)
    vals = bf16_to_f64(bits)
    m = vals.min(axis=1, keepdims=True)
    M = vals.max(axis=1, keepdims=True)
    lo_level = (3 * m + M) / 4
    hi_level = (m + 3 * M) / 4
    rec = np.where(codes == 1, hi_level, lo_level)
    assert np.all(np.abs(vals - rec) <= (M - m) / 4 * (1 + 1e-12))
    assert np.array_equal(codes == 1, 2 * (vals - m) > (M - m))
    # stored levels are the binary16 roundings of z and s
    z = f16_to_f64(offset)[:, None]
    s = f16_to_f64(scale)[:, None]
    assert np.all(np.abs(z - lo_level) <= np.maximum(np.abs(lo_level) * 2.0 ** -11, 2.0 ** -25))
    assert np.all(np.abs(s - (M - m) / 2) <= (M - m) / 2 * 2.0 ** -11)
    # exact midpoint rounds half-to-even to code 0; constant group keeps origin
    c, s1, o1 = quantize_groups_midpoint(bf([0.0, 1.0, 2.0, 0.5, 1.5])[None, :])
    assert c[0].tolist() == [0, 0, 1, 0, 1]
    assert f16_fraction(int(s1[0])) == 1 and f16_fraction(int(o1[0])) == Fraction(1, 2)
    c, s2, o2 = quantize_groups_midpoint(bf([7.0] * 5)[None, :])
    assert not c.any() and s2[0] == 0 and f16_fraction(int(o2[0])) == 7


def test_f16_metadata_rounding_pins():
    """IEEE binary16 facts the metadata rounding must reproduce: the largest
    finite value, the overflow threshold (ties to even go to infinity),
    subnormal ties, and +0.0 for results that round to zero."""
    from oracle.numerics import rn_f16_meta_bits
    assert rn_f16_meta_bits(Fraction(65504)) == 0x7BFF
    assert rn_f16_meta_bits(Fraction(65519)) == 0x7BFF
    assert rn_f16_meta_bits(Fraction(65520)) == 0x7C00          # tie -> even -> infinity
    assert rn_f16_meta_bits(Fraction(-70000)) == 0xFC00
    assert rn_f16_meta_bits(Fraction(1, 1 << 24)) == 0x0001      # smallest subnormal
    assert rn_f16_meta_bits(Fraction(1, 1 << 25)) == 0            # tie -> even (zero)
    assert rn_f16_meta_bits(Fraction(-1, 1 << 25)) == 0           # stored as +0.0
    assert rn_f16_meta_bits(Fraction(3, 1 << 25)) == 0x0002      # tie between 1 and 2 quanta -> 2
    assert rn_f16_meta_bits(Fraction(1, 3)) == 0x3555
    assert f16_fraction(0x3555) == Fraction(1365, 4096)
    # a group reaching beyond the binary16 range stores an infinite offset / scale
    codes, scale, offset = quantize_groups(bf([-131072.0, 0.0, 131072.0, 5.0])[None, :], 2)
    assert offset[0] == 0xFC00 and scale[0] == 0x7C00
    assert codes[0].tolist() == [0, 2, 3, 2]
