"""Pins of the oracle's QJL sketch.

* Lemma 3.2 (unbiasedness): the mean of Prod_QJL over many Gaussian S is
  <q, k> within a 4-sigma Monte Carlo band;
* Lemma 3.5 (distortion): with m >= 4/3 (1+eps)/eps^2 log(2/delta) the
  empirical rate of |Prod - <q,k>| > eps |q||k| is at most delta;
* the moment identity of the proof, E|z_i| and E z_i^2 for
  z_i = sqrt(pi/2) |k| s_i.q sign(s_i.k);
* exact sign bits (sign(0) = +1) and correctly rounded binary16 norms;
* the score estimator equals the definition on the stored bits and norms.
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
