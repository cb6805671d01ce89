"""Precision selection at prefill (oracle).

MixKVQ (page "方法细节", salience score; "MixKVQ的系统级实现细节" for GQA):
A_d = I_d * S_d with I_d the mean |Q_{t,d}| over the L_q prefill queries of all
query heads sharing the KV head, and S_d = (max k_d - min k_d)/(2^B - 1) over
the Key tokens being quantized. Channels are split into BF16 / UINT4 / UINT2
tiers by A_d (thresholds tau_BF16 > tau_UINT4). The workloads here fix the
tier sizes instead of the thresholds (12.5/25/62.5 % in the tiny workload,
1/12/115 channels for "~2.3 bits"), so the tiers are taken by rank of A_d:
the n16 highest channels are BF16, the next n4 are UINT4, the rest UINT2.
Ties are broken towards the lower channel index (the pages are silent).
The threshold form of the rule (mixkvq_threshold_select) compares A_d itself
with tau_BF16 and tau_UINT4.

Exactness. The mean and the 1/(2^B - 1) factor are positive constants common
to every channel of a KV head and do not change the ranking, so the rank key
is SQ_d * range_d with SQ_d the plain sum of |Q| and range_d = max - min. To
make the sum independent of summation order, every |q| is first put on a
fixed grid: psi(x) = round_half_even(x * 2^64) as an integer (exact for every
|q| >= 2^-56; smaller values move by at most 2^-65). Sums of psi are exact
integers and the products are compared exactly.

PN-Mix (page "核心公式", Eq.6): sigma_{h,i} = mean over the group's query heads
of E_t ||q_{h',t,i}||_2 times E_s ||k_{h,s,i}||_2, with i a RoPE pair: (i, i+64)
for the half-split layout of Llama-style models, (2i, 2i+1) for the adjacent
layout (page "背景与主要改动"). The top floor(r*D/2) pairs (32 at r = 0.5) are
kept at high precision, chosen once per KV head. Each pair norm is the
correctly rounded float64 sqrt(fl64(a^2 + b^2)) (a^2, b^2 are exact in
float64), put on the same psi grid and summed exactly; the common mean factors
are dropped for ranking, ties go to the lower pair index.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .numerics import bf16_to_f64

D = 128
TIER_U2, TIER_U4, TIER_BF16 = 0, 1, 2
_TWO64 = float(2 ** 64)


def psi_sum(values_f64: np.ndarray, axis) -> np.ndarray:
    """Exact integer sum of round_half_even(v * 2^64) along ``axis``.

    Returns a Python-int object array."""
    v = np.asarray(values_f64, dtype=np.float64)
    if np.any(v < 0) or np.any(v >= 2.0 ** 31):
        raise ValueError("psi grid needs 0 <= value < 2^31")
    g = np.rint(v * _TWO64)                  # exact integers held in f64
    c2 = np.floor(g / 2.0 ** 64)
    rest = g - c2 * 2.0 ** 64
    c1 = np.floor(rest / 2.0 ** 32)
    c0 = rest - c1 * 2.0 ** 32               # every chunk in [0, 2^32), exact
    s2 = c2.astype(np.int64).sum(axis=axis)
    s1 = c1.astype(np.int64).sum(axis=axis)
    s0 = c0.astype(np.int64).sum(axis=axis)
    out = np.empty(s0.shape, dtype=object)
    for idx in np.ndindex(s0.shape):
        out[idx] = (int(s2[idx]) << 64) + (int(s1[idx]) << 32) + int(s0[idx])
    return out


def _rank_desc(keys) -> np.ndarray:
    """rank[i] = number of entries with a larger key, or an equal key and a
    lower index."""
    n = len(keys)
    order = sorted(range(n), key=lambda i: (-keys[i], i))
    rank = np.empty(n, dtype=np.int64)
    for pos, i in enumerate(order):
        rank[i] = pos
    return rank


def query_sums(q_bits: np.ndarray) -> list:
    """SQ_d = sum of psi(|q_d|) over every query row given (all heads of a
    GQA group, any number of tokens), as exact Python ints. Sums of several
    calls add: this is the running query-magnitude accumulator of the MixKVQ
    system section (one decode query added per step)."""
    q = np.abs(bf16_to_f64(q_bits)).reshape(-1, D)
    sq = psi_sum(q, axis=0)
    return [int(sq[d]) for d in range(D)]


def mixkvq_keys_from_sums(sq, k_bits: np.ndarray):
    """Exact rank keys SQ_d * range_d (Fractions, units of 2^-64) from given
    query sums and the Key tokens [L_k, D] (bf16 bits) to be quantized."""
    k = bf16_to_f64(k_bits)
    rng = [Fraction(float(k[:, d].max())) - Fraction(float(k[:, d].min())) for d in range(D)]
    return [Fraction(int(sq[d])) * rng[d] for d in range(D)]


def mixkvq_keys(q_bits: np.ndarray, k_bits: np.ndarray):
    """Exact rank keys for one KV head.

    q_bits: [g, L_q, D] bf16 bits of the group's prefill queries.
    k_bits: [L_k, D] bf16 bits of the Key tokens to be quantized.
    Returns list of Fractions SQ_d * range_d (units of 2^-64)."""
    return mixkvq_keys_from_sums(query_sums(q_bits), k_bits)


def mixkvq_select_sums(sq, k_bits, n16: int, n4: int):
    """Per-flush reselection (MixKVQ: I_d and S_d refreshed every R tokens;
    the running accumulator of query magnitudes): the tiers of one page from
    the accumulated query sums and the page's own Key tokens. Returns as
    mixkvq_select."""
    return _select_from_keys(mixkvq_keys_from_sums(sq, k_bits), n16, n4)


def mixkvq_select(q_bits, k_bits, n16: int, n4: int):
    """Tier of every channel and the channel order (BF16, UINT4, UINT2 tiers,
    each ascending by channel index) for one KV head."""
    return _select_from_keys(mixkvq_keys(q_bits, k_bits), n16, n4)


def _select_from_keys(keys, n16: int, n4: int):
    rank = _rank_desc(keys)
    tier = np.where(rank < n16, TIER_BF16, np.where(rank < n16 + n4, TIER_U4, TIER_U2))
    perm = np.concatenate([np.nonzero(tier == t)[0] for t in (TIER_BF16, TIER_U4, TIER_U2)])
    return tier.astype(np.uint8), perm.astype(np.uint8), rank


def mixkvq_salience(q_bits, k_bits):
    """A_d = I_d * S_d of every channel, as exact Fractions (MixKVQ
    "方法细节"): I_d = mean over the g * L_q prefill query rows of |Q_{t,d}|
    (each |q| on the 2^-64 grid of query_sums), S_d = (max k_d - min k_d) /
    (2^B - 1) with B = 2.

    q_bits: [g, L_q, D] bf16 bits; k_bits: [L_k, D] bf16 bits."""
    q_bits = np.asarray(q_bits)
    rows = q_bits.shape[0] * q_bits.shape[1]
    sq = query_sums(q_bits)
    k = bf16_to_f64(k_bits)
    out = []
    for d in range(D):
        i_d = Fraction(sq[d], 2 ** 64 * rows)
        s_d = (Fraction(float(k[:, d].max())) - Fraction(float(k[:, d].min()))) / 3
        out.append(i_d * s_d)
    return out


def mixkvq_threshold_select(q_bits, k_bits, cap16: int, cap4: int, tau_bf16: float, tau_u4: float):
    """Tiers by the salience thresholds (MixKVQ three-tier rule, Algorithm 1's
    tau_BF16 and tau_UINT4): A_d > tau_bf16 is BF16, tau_u4 < A_d <= tau_bf16
    is UINT4, the rest UINT2 (so the UINT4 tier is empty when tau_bf16 <=
    tau_u4). The comparisons are exact. Reading for storage with a fixed
    page size: at most cap16 BF16 and cap4 UINT4 channels per head; a tier
    given more channels keeps its highest-ranked ones (the COUNT ranking) and
    the rest move down one tier. Returns (tier, perm, rank, n16, n4)."""
    A = mixkvq_salience(q_bits, k_bits)
    keys = mixkvq_keys(q_bits, k_bits)
    rank = _rank_desc(keys)
    t16, t4 = Fraction(tau_bf16), Fraction(tau_u4)
    above16 = [A[d] > t16 for d in range(D)]
    above4 = [A[d] > t4 and not above16[d] for d in range(D)]
    by_rank = sorted(range(D), key=lambda d: rank[d])
    bf16 = [d for d in by_rank if above16[d]][:cap16]
    cand4 = [d for d in by_rank if (above16[d] and d not in bf16) or above4[d]]
    u4 = cand4[:cap4]
    tier = np.full(D, TIER_U2, dtype=np.uint8)
    tier[bf16] = TIER_BF16
    tier[u4] = TIER_U4
    perm = np.concatenate([np.nonzero(tier == t)[0] for t in (TIER_BF16, TIER_U4, TIER_U2)])
    return tier, perm.astype(np.uint8), rank, len(bf16), len(u4)


def record_counts(rec) -> tuple:
    """(BF16, UINT4) channel counts held in a record's 2-bit tier codes."""
    rec = np.asarray(rec, np.uint8)
    codes = [(int(rec[D + d // 4]) >> (2 * (d % 4))) & 3 for d in range(D)]
    return codes.count(TIER_BF16), codes.count(TIER_U4)


def mixkvq_record(tier: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """160-byte selection record: perm[128] then 2-bit tier codes, low bits
    first (channel d at byte d//4, bits 2*(d%4))."""
    rec = np.zeros(160, np.uint8)
    rec[:128] = perm
    for d in range(D):
        rec[128 + d // 4] |= int(tier[d]) << (2 * (d % 4))
    return rec


def pair_channels(layout: str):
    i = np.arange(D // 2)
    if layout == "half":
        return i, i + D // 2
    return 2 * i, 2 * i + 1


def _pair_norms(x_f64: np.ndarray, layout: str) -> np.ndarray:
    a, b = pair_channels(layout)
    return np.sqrt(x_f64[..., a] * x_f64[..., a] + x_f64[..., b] * x_f64[..., b])


def pnmix_keys(q_bits, k_bits, layout: str = "half"):
    """Exact integer pair scores (QN_i * KN_i) for one KV head.

    q_bits [g, L_q, D], k_bits [L_k, D]."""
    qn = psi_sum(_pair_norms(bf16_to_f64(q_bits), layout).reshape(-1, D // 2), axis=0)
    kn = psi_sum(_pair_norms(bf16_to_f64(k_bits), layout).reshape(-1, D // 2), axis=0)
    return [int(qn[i]) * int(kn[i]) for i in range(D // 2)]


def pnmix_select(q_bits, k_bits, n_hi_pairs: int = 32, layout: str = "half"):
    """Returns (pair mask bool [64], high-channel mask bool [128], 8-byte record)."""
    keys = pnmix_keys(q_bits, k_bits, layout)
    rank = _rank_desc(keys)
    pair_hi = rank < n_hi_pairs
    a, b = pair_channels(layout)
    ch = np.zeros(D, dtype=bool)
    ch[a[pair_hi]] = True
    ch[b[pair_hi]] = True
    rec = np.zeros(8, np.uint8)
    for i in range(D // 2):
        if pair_hi[i]:
            rec[i // 8] |= 1 << (i % 8)
    return pair_hi, ch, rec


def hi_channels_from_record(rec, layout: str = "half") -> np.ndarray:
    rec = np.asarray(rec, np.uint8)
    a, b = pair_channels(layout)
    ch = np.zeros(D, dtype=bool)
    for i in range(D // 2):
        if (int(rec[i // 8]) >> (i % 8)) & 1:
            ch[a[i]] = True
            ch[b[i]] = True
    return ch
