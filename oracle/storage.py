"""Storage accounting (oracle).

KIVI blog section 7: per layer, per KV head and per request the cache costs
M = D [ (2T - r_K - r_V)(b/8 + 2e/G) + (r_K + r_V) f ] bytes, with T visible
tokens, r_K/r_V the full-precision residual lengths, b code bits, e bytes per
origin or step, f bytes per float; unquantized it is 2 T D f.

PN-Mix page ("核心公式", Appendix G and the measured results): persistent bytes
are sinks + residual (K and V, full precision) + the LSB plane of every Key
channel + the upper-2-bit plane of the high channels + per-channel Key
scale/offset per page + 2-bit Value codes + per-token Value scale/offset per
32-channel group + the pair mask stored once as bits; "about 2.26 bit" is the
average Key storage at 32K quantized tokens with the residual excluded.

MixKVQ ("MixKVQ的系统级实现细节"): quantized codes, BF16 salient channels and
the residual buffer; B_eff is the mean code width over channels (threshold
search paragraph).
"""
from __future__ import annotations

from fractions import Fraction


def kivi_bytes(T, D, G, r_k, r_v, b, e, f):
    """Exact bytes of the KIVI-form formula (a Fraction)."""
    return Fraction(D) * ((2 * T - r_k - r_v) * (Fraction(b, 8) + Fraction(2 * e, G)) + (r_k + r_v) * f)


def kivi_bits_per_element(b, e, G):
    """Average bits of a quantized element: b + 2*8e/G."""
    return b + Fraction(2 * 8 * e, G)


def pnmix_breakdown(*, h_kv_d, n_sink, n_quant, n_resid, r=Fraction(1, 2), G=128, G_V=32,
                    b_hi=3, b_lo=1, v_bits=2, float_bytes=2):
    """Persistent PN-Mix cache bytes by region (one layer, one request).

    h_kv_d = KV heads x head_dim (channels); n_quant a multiple of G."""
    C = h_kv_d
    n_hi = int(r * C)            # channels of the selected pairs (floor(r d / 2) pairs)
    pages = n_quant // G
    out = {
        "sink": 2 * n_sink * C * float_bytes,
        "residual": 2 * n_resid * C * float_bytes,
        "k_codes": (n_quant * C * b_lo + n_quant * n_hi * (b_hi - b_lo)) // 8,
        "k_meta": pages * C * 2 * float_bytes,
        "v_codes": n_quant * C * v_bits // 8,
        "v_meta": n_quant * (C // G_V) * 2 * float_bytes,
        "mask": (C // 2 + 7) // 8,
    }
    out["total"] = sum(out.values())
    return out


def pnmix_key_bits(*, d, n_quant, n_sink, r=Fraction(1, 2), G=128, b_hi=3, b_lo=1, meta_bits=32, sink_bits=16):
    """Average Key storage bits per element over quantized + sink tokens
    (residual excluded): codes r*b_hi + (1-r)*b_lo plus 32 metadata bits per
    channel per G-token group, sinks at 16 bits."""
    per_quant = r * b_hi + (1 - r) * b_lo + Fraction(meta_bits, G)
    return (n_quant * per_quant + n_sink * sink_bits) / Fraction(n_quant + n_sink)


def mixkvq_breakdown(*, n_kv_heads, d, n16, n4, n_quant, n_resid, G=128, G_V=32, v_bits=2, e=2, f=2,
                     per_page_records=False):
    """Logical persistent bytes of the MixKVQ cache for one layer/request:
    per page and KV head, BF16 channels at f bytes/token, UINT4/UINT2 codes,
    one scale + offset (e bytes each) per quantized channel; Values at
    v_bits with one scale + offset per token per G_V channels; the BF16
    residual for K and V; the selection record (channel order + tiers), one
    per KV head, or one per page when the tiers are re-selected at every
    flush."""
    n2 = d - n16 - n4
    pages = n_quant // G
    H = n_kv_heads
    out = {
        "k_bf16": H * n_quant * n16 * f,
        "k_codes": H * n_quant * (4 * n4 + 2 * n2) // 8,
        "k_meta": H * pages * (n4 + n2) * 2 * e,
        "v_codes": H * n_quant * d * v_bits // 8,
        "v_meta": H * n_quant * (d // G_V) * 2 * e,
        "residual": H * 2 * n_resid * d * f,
        "mask": H * (pages if per_page_records else 1) * (d + d // 4),
    }
    out["total"] = sum(out.values())
    return out


def mixkvq_beff(d, n16, n4):
    """Mean code width over channels (MixKVQ's B_eff)."""
    n2 = d - n16 - n4
    return Fraction(16 * n16 + 4 * n4 + 2 * n2, d)
