"""Pins of the oracle's QJL sketch.

* Lemma 3.2 (unbiasedness): the mean of Prod_QJL over many Gaussian S is
  <q, k> within a 4-sigma Monte Carlo band;
* Lemma 3.5 (distortion): with m >= 4/3 (1+eps)/eps^2 log(2/delta) the
  empirical rate of |Prod - <q,k>| > eps |q||k| is at most delta;
* the moment identity of the proof, E|z_i| and E z_i^2 for
  z_i = sqrt(pi/2) |k| s_i.q sign(s_i.k);
* exact sign bits (sign(0) = +1) and correctly rounded binary16 norms;
* the score estimator equals the definition on the stored bits and norms;
* the outlier split ("处理异常值"): outlier channels are the largest exact
  sums of |K| (constructed outliers found, ties to the lower channel, brute
  force over Fractions); the split estimator is unbiased (a wrong instance
  factor or norm makes it biased) and has a smaller error than one instance
  when a few channels dominate the key norm (the distortion of Theorem 3.6
  grows with the norm); with all outlier coordinates zero the normal
  instance's bits and norm are plain QJL's and the outlier instance reads
  +1 with norm 0; the packed page round-trips.
"""
import math
from fractions import Fraction

import numpy as np

from oracle import qjl
from oracle.numerics import bf16_fraction, f16_to_f64, rn_f16_bits


def test_unbiased_monte_carlo():
    rng = np.random.default_rng(0)
    d, m, trials = 8, 16, 60000
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    S = rng.standard_normal((trials, m, d))
    sq = np.einsum("tmd,d->tm", S, q)
    sk = np.einsum("tmd,d->tm", S, k)
    prods = math.sqrt(math.pi / 2) / m * np.linalg.norm(k) * np.sum(sq * np.where(sk >= 0, 1.0, -1.0), axis=1)
    mean, sd = prods.mean(), prods.std() / math.sqrt(trials)
    assert abs(mean - q @ k) < 4 * sd
    # the estimator of one draw matches the helper
    assert abs(qjl.prod_qjl(q, k, S[0]) - prods[0]) < 1e-12


def test_distortion_bound():
    rng = np.random.default_rng(1)
    d, eps, delta = 16, 0.5, 0.1
    m = math.ceil(4 / 3 * (1 + eps) / eps ** 2 * math.log(2 / delta))
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    trials = 20000
    S = rng.standard_normal((trials, m, d))
    sq = S @ q
    sk = S @ k
    prods = math.sqrt(math.pi / 2) / m * np.linalg.norm(k) * np.sum(sq * np.where(sk >= 0, 1.0, -1.0), axis=1)
    rate = np.mean(np.abs(prods - q @ k) > eps * np.linalg.norm(q) * np.linalg.norm(k))
    assert rate <= delta


def test_moments_of_single_term():
    rng = np.random.default_rng(2)
    d, n = 6, 400000
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    s = rng.standard_normal((n, d))
    z = math.sqrt(math.pi / 2) * np.linalg.norm(k) * (s @ q) * np.where(s @ k >= 0, 1.0, -1.0)
    nq, nk = np.linalg.norm(q), np.linalg.norm(k)
    for ell in (1, 2):
        expect = (math.sqrt(math.pi) * nk * nq) ** ell * math.gamma((ell + 1) / 2) / math.sqrt(math.pi)
        got = np.mean(np.abs(z) ** ell)
        assert abs(got - expect) < 0.02 * expect


def test_exact_signs_and_norms():
    rng = np.random.default_rng(3)
    S = (rng.standard_normal((64, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    K = (rng.standard_normal((20, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    K[0] = 0                                         # zero key: all signs +1, norm 0
    K[1] = 0
    K[1, 0] = 0x4040                                 # 3.0
    K[1, 1] = 0x4080                                 # 4.0  -> norm exactly 5
    bits = qjl.sketch_bits(S, K)
    for i in range(0, 64, 7):
        for t in range(20):
            exact = sum((bf16_fraction(int(a)) * bf16_fraction(int(b)) for a, b in zip(S[i], K[t])), Fraction(0))
            assert bits[i, t] == (1 if exact >= 0 else 0)
    assert np.all(bits[:, 0] == 1)
    norms = qjl.key_norms(K)
    assert norms[0] == 0 and f16_to_f64(norms[1:2])[0] == 5.0
    # correctly rounded: |nu - ||k||| is at most half an ulp, decided on squares
    for t in range(2, 20):
        ssum = sum((bf16_fraction(int(b)) ** 2 for b in K[t]), Fraction(0))
        v = Fraction(f16_to_f64(norms[t:t + 1])[0])
        e = math.floor(math.log2(v))
        half_ulp = Fraction(2) ** (e - 10) / 2
        assert (v - half_ulp) ** 2 <= ssum <= (v + half_ulp) ** 2


def test_estimator_on_stored_sketch():
    rng = np.random.default_rng(4)
    S = (rng.standard_normal((256, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    K = (rng.standard_normal((30, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q = rng.standard_normal(128)
    bits = qjl.sketch_bits(S, K)
    norms = qjl.key_norms(K)
    est = qjl.estimate_scores(q, S, bits, norms)
    from oracle.numerics import bf16_to_f64
    Sf = bf16_to_f64(S)
    for t in range(30):
        signs = np.where(bits[:, t] == 1, 1.0, -1.0)
        val = math.sqrt(math.pi / 2) / 256 * f16_to_f64(norms[t:t + 1])[0] * float((Sf @ q) @ signs)
        assert abs(val - est[t]) <= 1e-12 * max(1.0, abs(val))
    assert rn_f16_bits(Fraction(5)) == 0x4500


# ------------------------------------------------------------------ outlier split
def _bf16_bits(x):
    import torch
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_outlier_channels_found_and_ties():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((300, 128))
    chans = [3, 17, 40, 41, 77, 90, 101, 127]
    k[:, chans] *= 20.0
    kb = _bf16_bits(k)
    outl = qjl.outlier_mask(kb, 8)
    assert sorted(np.nonzero(outl)[0].tolist()) == chans
    # brute force: exact Fraction sums, sorted by (-sum, channel)
    small = _bf16_bits(rng.standard_normal((7, 128)))
    sums = [sum(abs(bf16_fraction(int(small[t, d]))) for t in range(7)) for d in range(128)]
    want = sorted(range(128), key=lambda d: (-sums[d], d))[:5]
    assert sorted(np.nonzero(qjl.outlier_mask(small, 5))[0].tolist()) == sorted(want)
    # equal sums: the lower channel wins
    tie = np.ones((4, 128), np.float32)
    tie[:, 60] = tie[:, 9] = 2.0
    tie[:, 100] = 2.0
    got = np.nonzero(qjl.outlier_mask(_bf16_bits(tie), 2))[0].tolist()
    assert got == [9, 60]
    rec = qjl.outlier_record(qjl.outlier_mask(_bf16_bits(tie), 3))
    assert rec[1] == 1 << 1 and rec[7] == 1 << 4 and rec[12] == 1 << 4 and rec.sum() == 2 + 16 + 16
    assert np.array_equal(qjl.outlier_mask_from_record(rec), qjl.outlier_mask(_bf16_bits(tie), 3))


def test_split_estimator_unbiased_and_tighter():
    rng = np.random.default_rng(6)
    d, m, m_o, trials = 16, 32, 16, 40000
    outl = np.zeros(d, bool)
    outl[[2, 11]] = True
    q = rng.standard_normal(d)
    q[outl] = [0.7, -0.9]                     # a query not aligned with the outliers
    k = rng.standard_normal(d)
    k[outl] *= 25.0
    split, plain = np.empty(trials), np.empty(trials)
    for t in range(trials):
        S_i = rng.standard_normal((m, d))
        S_o = rng.standard_normal((m_o, d))
        split[t] = qjl.prod_qjl_split(q, k, S_i, S_o, outl)
        plain[t] = qjl.prod_qjl(q, k, np.concatenate([S_i, S_o]))
    mean, sd = split.mean(), split.std() / math.sqrt(trials)
    assert abs(mean - q @ k) < 4 * sd
    # closed-form variance (the moment identity E z^2 = pi/2 |q|^2 |k|^2 of
    # each term, per instance): a wrong factor or norm moves it
    def var(qq, kk, rows):
        return (math.pi / 2 * (qq @ qq) * (kk @ kk) - (qq @ kk) ** 2) / rows
    q_i, k_i = np.where(outl, 0.0, q), np.where(outl, 0.0, k)
    want = var(q_i, k_i, m) + var(np.where(outl, q, 0.0), np.where(outl, k, 0.0), m_o)
    assert abs(np.var(split) / want - 1) < 0.06
    # one instance of the same total rows: the outlier norm inflates its error
    assert np.mean((split - q @ k) ** 2) < 0.5 * np.mean((plain - q @ k) ** 2)
    # a wrong outlier-instance factor (1/m instead of 1/m_o) is biased
    q_o, k_o = np.where(outl, q, 0.0), np.where(outl, k, 0.0)
    wrong = np.array([qjl.prod_qjl(np.where(outl, 0, q), np.where(outl, 0, k), rng.standard_normal((m, d)))
                      + qjl.prod_qjl(q_o, k_o, rng.standard_normal((m_o, d))) * m_o / m for _ in range(4000)])
    assert abs(wrong.mean() - q @ k) > 4 * wrong.std() / math.sqrt(4000)


def test_split_sketch_reduces_and_page_roundtrip():
    from oracle import flush, layout
    rng = np.random.default_rng(7)
    m, m_o = 128, 64
    s = _bf16_bits(rng.standard_normal((m + m_o, 128)))
    outl = np.zeros(128, bool)
    outl[[5, 6, 70, 99]] = True
    k = rng.standard_normal((128, 128))
    k[:, outl] = 0.0
    kb = _bf16_bits(k)
    bits, nu_i, nu_o = qjl.split_sketch(s, m, kb, outl)
    assert np.array_equal(bits[:m], qjl.sketch_bits(s[:m], kb))
    assert np.array_equal(nu_i, qjl.key_norms(kb))
    assert np.all(bits[m:] == 1) and np.all(nu_o == 0)
    # nonzero outliers: each instance sees only its own coordinates
    k2 = rng.standard_normal((128, 128))
    k2[:, outl] *= 30.0
    kb2 = _bf16_bits(k2)
    bits2, nu_i2, nu_o2 = qjl.split_sketch(s, m, kb2, outl)
    S = bf16_to_f64_(s)
    K = bf16_to_f64_(kb2)
    assert np.array_equal(bits2[m:], ((S[m:][:, outl] @ K[:, outl].T) >= 0).astype(np.uint8))
    assert np.array_equal(bits2[:m], ((S[:m][:, ~outl] @ K[:, ~outl].T) >= 0).astype(np.uint8))
    assert np.allclose(f16_to_f64(nu_o2), np.linalg.norm(K[:, outl], axis=1), rtol=1e-3)
    v = _bf16_bits(rng.standard_normal((128, 128)))
    page = flush.flush_qjl_page(kb2, v, s, m=m, outl=outl)
    g = layout.qjl_geometry(m, m_o)
    assert page.shape[0] == g["stride"] and g["off_v"] == 16 * (m + m_o) + 512
    u = layout.unpack_qjl_page(page, m, m_o)
    assert np.array_equal(u["bits"][:m + m_o], bits2)
    assert np.array_equal(u["norms"], nu_i2) and np.array_equal(u["norms_out"], nu_o2)
    # the estimator on the stored page equals the split definition
    q = rng.standard_normal(128)
    est = qjl.estimate_scores_split(q, s, m, outl, u["bits"][:m + m_o], u["norms"], u["norms_out"])
    want = (math.sqrt(math.pi / 2) / m * f16_to_f64(nu_i2) * ((S[:m][:, ~outl] @ q[~outl]) @ (2.0 * bits2[:m] - 1))
            + math.sqrt(math.pi / 2) / m_o * f16_to_f64(nu_o2) * ((S[m:][:, outl] @ q[outl]) @ (2.0 * bits2[m:] - 1)))
    assert np.allclose(est, want, rtol=1e-12, atol=1e-12)


def bf16_to_f64_(bits):
    from oracle.numerics import bf16_to_f64
    return bf16_to_f64(bits)
