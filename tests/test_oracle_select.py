"""Pins of the oracle's precision selection.

* MixKVQ query awareness (page "速读" and "背景知识与关键观察", error-only
  ablation in the appendix): on the tiny workload the four outlier Key
  channels whose query is NOT attenuated hold the top saliency ranks (they are
  BF16 tier), the four attenuated ones fall below every normal channel in
  A_d, while an error-only ranking (A_d = S_d) puts all eight first;
* ranking agrees with a brute-force Fraction computation of
  mean|Q| * (max k - min k)/3 (the psi grid is exact for these inputs);
* ties go to the lower index; the record encodes order and tiers;
* PN-Mix Eq.6: ranking agrees with float64 means of pair norms when there is
  no near tie, is invariant to token order, and a zero-Key pair ranks last;
  the adjacent and half-split layouts pair the right channels.
* Per-flush reselection (MixKVQ's running query-magnitude accumulator, tiers
  refreshed at every flush): query sums accumulate exactly (chunked sums of
  integers on the 2^-64 grid equal the one-shot sum; 1.0 counts 2^64); with
  equal query sums the page's Key ranges alone order the channels, with
  equal ranges the sums alone; a page's tiers follow its own Keys.
"""
from fractions import Fraction

import numpy as np

import kvq_synth as synth
from oracle import select
from oracle.numerics import bf16_fraction, bf16_to_f64


def tiny_inputs():
    w = synth.WORKLOADS["tiny_mixkvq"]
    q, k, _ = synth.prefill(w, "cpu")
    qb = synth.bf16_bits(q)[0]                           # [g, Lq, D]
    kb = synth.bf16_bits(k)[0, 0, : w.n_pages * 128]     # [Lk, D]
    return w, qb, kb, synth.outlier_channels(w)[0, 0]


def test_query_aware_tiers_on_tiny_workload():
    w, qb, kb, oc = tiny_inputs()
    tier, perm, rank = select.mixkvq_select(qb, kb, w.n_bf16, w.n_u4)
    plain, attenuated = oc[4:], oc[:4]
    assert set(rank[plain].tolist()) == {0, 1, 2, 3}
    assert np.all(tier[plain] == select.TIER_BF16)
    normal = np.setdiff1d(np.arange(128), oc)
    keys = select.mixkvq_keys(qb, kb)
    assert max(keys[c] for c in attenuated) < min(keys[c] for c in normal)
    # error-only ablation: rank by range alone puts all eight outliers first
    k = bf16_to_f64(kb)
    rng = k.max(axis=0) - k.min(axis=0)
    assert set(np.argsort(-rng, kind="stable")[:8].tolist()) == set(oc.tolist())
    # tier sizes and channel order
    assert (tier == select.TIER_BF16).sum() == 16 and (tier == select.TIER_U4).sum() == 32
    assert sorted(perm.tolist()) == list(range(128))
    assert np.all(tier[perm[:16]] == 2) and np.all(tier[perm[16:48]] == 1) and np.all(tier[perm[48:]] == 0)
    for lo, hi in ((0, 16), (16, 48), (48, 128)):
        assert np.all(np.diff(perm[lo:hi].astype(int)) > 0)


def test_mixkvq_rank_matches_fraction_brute_force():
    rng = np.random.default_rng(4)
    g, Lq, Lk = 2, 9, 11
    q = (rng.standard_normal((g, Lq, 128)) * rng.uniform(0.1, 3, 128)).astype(np.float32)
    k = (rng.standard_normal((Lk, 128)) * rng.uniform(0.1, 3, 128)).astype(np.float32)
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    A = []
    for d in range(128):
        imp = sum(abs(bf16_fraction(int(x))) for x in qb[:, :, d].ravel()) / (g * Lq)
        col = [bf16_fraction(int(x)) for x in kb[:, d]]
        A.append(imp * (max(col) - min(col)) / 3)
    expect = sorted(range(128), key=lambda d: (-A[d], d))
    _, _, rank = select.mixkvq_select(qb, kb, 8, 24)
    assert [int(np.nonzero(rank == r)[0][0]) for r in range(128)] == expect


def test_ties_go_to_lower_channel_and_record():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 4, 128)).astype(np.float32)
    k = rng.standard_normal((6, 128)).astype(np.float32)
    q[:, :, 9] = q[:, :, 3] * 0 + 50.0
    q[:, :, 3] = 50.0
    k[:, 9] = k[:, 3]
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    tier, perm, rank = select.mixkvq_select(qb, kb, 1, 1)
    assert rank[3] == 0 and rank[9] == 1
    rec = select.mixkvq_record(tier, perm)
    assert rec[0] == 3 and rec[1] == 9
    assert (rec[128 + 3 // 4] >> (2 * (3 % 4))) & 3 == select.TIER_BF16
    assert (rec[128 + 9 // 4] >> (2 * (9 % 4))) & 3 == select.TIER_U4


def test_pnmix_ranking_float_means_and_invariance():
    rng = np.random.default_rng(6)
    g, Lq, Lk = 4, 40, 50
    scale = rng.uniform(0.2, 2.0, 128)
    q = (rng.standard_normal((g, Lq, 128)) * scale).astype(np.float32)
    k = (rng.standard_normal((Lk, 128)) * scale[::-1]).astype(np.float32)
    k[:, 5] = 0.0
    k[:, 69] = 0.0            # pair 5 of the half-split layout has a zero Key
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    for layout in ("half", "adjacent"):
        a, b = select.pair_channels(layout)
        qf, kf = bf16_to_f64(qb), bf16_to_f64(kb)
        qn = np.sqrt(qf[..., a] ** 2 + qf[..., b] ** 2).reshape(-1, 64).mean(axis=0)
        kn = np.sqrt(kf[..., a] ** 2 + kf[..., b] ** 2).mean(axis=0)
        sigma = qn * kn
        srt = np.sort(sigma)[::-1]
        assert srt[31] - srt[32] > 1e-9 * srt[31]          # no near tie at the cut
        pair_hi, ch, rec = select.pnmix_select(qb, kb, 32, layout)
        assert set(np.nonzero(pair_hi)[0].tolist()) == set(np.argsort(-sigma)[:32].tolist())
        assert ch.sum() == 64 and np.array_equal(select.hi_channels_from_record(rec, layout), ch)
        perm_t = rng.permutation(Lk)
        keys1 = select.pnmix_keys(qb, kb, layout)
        keys2 = select.pnmix_keys(qb[:, ::-1], kb[perm_t], layout)
        assert keys1 == keys2                                  # exact, order independent
    keys = select.pnmix_keys(qb, kb, "half")
    assert keys[5] == 0 and min(keys) == 0
    assert select.pair_channels("half")[1][5] == 69 and select.pair_channels("adjacent")[1][5] == 11


def _bf16(x):
    return synth.bf16_bits(__import__("torch").tensor(np.asarray(x, np.float32)).to(__import__("torch").bfloat16))


def test_query_sums_accumulate_exactly():
    rng = np.random.default_rng(5)
    q = _bf16(rng.standard_normal((3, 40, 128)) * 4.0)
    whole = select.query_sums(q)
    parts = [select.query_sums(q[:, :13]), select.query_sums(q[:, 13:29]), select.query_sums(q[:, 29:])]
    assert whole == [a + b + c for a, b, c in zip(*parts)]
    ones = _bf16(np.ones((2, 3, 128)))
    assert select.query_sums(ones) == [6 * 2 ** 64] * 128     # psi(1.0) = 2^64, six rows
    half = _bf16(np.full((1, 1, 128), -0.5))
    assert select.query_sums(half) == [2 ** 63] * 128          # magnitudes: |-0.5| = 2^-1


def test_reselect_orders_by_range_with_equal_sums():
    n16, n4 = 3, 10
    sq = [2 ** 64] * 128
    k = np.zeros((128, 128), np.float32)
    k[1, :] = np.arange(128) + 1.0                               # range of channel d = d + 1
    tier, perm, rank = select.mixkvq_select_sums(sq, _bf16(k), n16, n4)
    assert list(rank) == [127 - d for d in range(128)]
    assert list(perm[:n16]) == [125, 126, 127]                   # largest ranges, ascending order
    assert list(perm[n16:n16 + n4]) == list(range(115, 125))
    assert list(perm[n16 + n4:]) == list(range(115))
    assert all(tier[d] == (2 if d >= 125 else 1 if d >= 115 else 0) for d in range(128))


def test_reselect_orders_by_sums_with_equal_ranges():
    n16, n4 = 2, 4
    sq = [(d % 7 + 1) * 2 ** 60 for d in range(128)]               # ties within each residue class
    k = np.zeros((128, 128), np.float32)
    k[5, :] = 2.0                                                 # every range 2
    tier, perm, rank = select.mixkvq_select_sums(sq, _bf16(k), n16, n4)
    top = [d for d in range(128) if d % 7 == 6]                   # the largest sum, lower index first
    assert list(perm[:n16]) == top[:n16]
    assert sorted(perm[n16:n16 + n4]) == list(perm[n16:n16 + n4]) and set(perm[n16:n16 + n4]) == set(top[n16:n16 + n4])


def test_reselect_follows_each_pages_keys():
    w, qb, kb, oc = tiny_inputs()
    sq = select.query_sums(qb)
    # the prefill selection is the reselection over all the prefill Keys
    t_all, p_all, _ = select.mixkvq_select(qb, kb, w.n_bf16, w.n_u4)
    t_s, p_s, _ = select.mixkvq_select_sums(sq, kb, w.n_bf16, w.n_u4)
    assert np.array_equal(p_all, p_s) and np.array_equal(t_all, t_s)
    # a page whose outlier channels were flattened loses them from the BF16 tier
    page = bf16_to_f64(kb[:128]).astype(np.float32)
    page[:, oc[4:]] = 0.0
    t_p, _, _ = select.mixkvq_select_sums(sq, _bf16(page), w.n_bf16, w.n_u4)
    assert all(t_p[d] == 0 for d in oc[4:])
    assert all(t_all[d] == 2 for d in oc[4:])


# ------------------------------------------------------------------ threshold tiers
# MixKVQ three-tier rule with the salience thresholds: A_d > tau_BF16 is
# BF16, tau_UINT4 < A_d <= tau_BF16 is UINT4, A_d <= tau_UINT4 is UINT2.

def _ramp_inputs():
    """Closed form: every |q| = 1 (I_d = 1), Keys 0 and (d + 1)/16 (range
    (d + 1)/16), so A_d = (d + 1)/48 exactly, over g = 2 heads, L_q = 4."""
    qb = np.full((2, 4, 128), 0x3F80, np.uint16)                      # bf16 1.0
    k = np.zeros((3, 128), np.float32)
    k[1] = (np.arange(128) + 1) / 16.0
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)                 # exact in bf16
    return qb, kb


def test_threshold_salience_closed_form():
    qb, kb = _ramp_inputs()
    A = select.mixkvq_salience(qb, kb)
    assert A == [Fraction(d + 1, 48) for d in range(128)]
    # tau_bf16 = 2.5 = A_119 exactly, tau_u4 = 2 = A_95 exactly: both
    # comparisons are strict on the upper side
    tier, perm, _, n16, n4 = select.mixkvq_threshold_select(qb, kb, 128, 128, 2.5, 2.0)
    expect = np.where(np.arange(128) >= 120, select.TIER_BF16, np.where(np.arange(128) >= 96, select.TIER_U4, select.TIER_U2))
    assert np.array_equal(tier, expect) and (n16, n4) == (8, 24)
    assert list(perm[:8]) == list(range(120, 128)) and list(perm[8:32]) == list(range(96, 120))
    assert select.record_counts(select.mixkvq_record(tier, perm)) == (8, 24)
    # capacities: the BF16 tier keeps its 4 best (127..124), the other 4 move
    # down to compete for the 10 UINT4 places with the 24 channels above 2
    tier, _, _, n16, n4 = select.mixkvq_threshold_select(qb, kb, 4, 10, 2.5, 2.0)
    assert (n16, n4) == (4, 10)
    assert set(np.nonzero(tier == select.TIER_BF16)[0]) == set(range(124, 128))
    assert set(np.nonzero(tier == select.TIER_U4)[0]) == set(range(114, 124))


def test_threshold_empty_uint4_tier_with_published_thresholds():
    # the MixKVQ page's R1-Qwen-14B thresholds (tau_BF16, tau_UINT4) = (1.52, 1.60):
    # tau_BF16 <= tau_UINT4 leaves no A_d with tau_UINT4 < A_d <= tau_BF16
    w, qb, kb, _ = tiny_inputs()
    A = select.mixkvq_salience(qb, kb)
    tier, _, _, n16, n4 = select.mixkvq_threshold_select(qb, kb, 128, 128, 1.52, 1.60)
    assert n4 == 0 and not np.any(tier == select.TIER_U4)
    assert n16 == sum(a > Fraction(1.52) for a in A)
    # the Llama-8B pair (1.44, 0.79) gives all three tiers on the outlier workload
    tier, _, _, n16, n4 = select.mixkvq_threshold_select(qb, kb, 128, 128, 1.44, 0.79)
    assert n16 == sum(a > Fraction(1.44) for a in A)
    assert n4 == sum(Fraction(0.79) < a <= Fraction(1.44) for a in A)


def test_threshold_between_ranks_reproduces_count_mode():
    w, qb, kb, _ = tiny_inputs()
    A = select.mixkvq_salience(qb, kb)
    tier_c, perm_c, rank = select.mixkvq_select(qb, kb, w.n_bf16, w.n_u4)
    by_rank = sorted(range(128), key=lambda d: rank[d])
    # A_d and the COUNT ranking key differ by a positive constant factor
    assert all(A[by_rank[i]] >= A[by_rank[i + 1]] for i in range(127))

    def between(i):   # a double strictly between the i-th and (i+1)-th salience
        hi, lo = A[by_rank[i]], A[by_rank[i + 1]]
        t = float((hi + lo) / 2)
        assert lo < Fraction(t) < hi
        return t
    t16, t4 = between(w.n_bf16 - 1), between(w.n_bf16 + w.n_u4 - 1)
    tier, perm, _, n16, n4 = select.mixkvq_threshold_select(qb, kb, 128, 128, t16, t4)
    assert (n16, n4) == (w.n_bf16, w.n_u4)
    assert np.array_equal(tier, tier_c) and np.array_equal(perm, perm_c)
