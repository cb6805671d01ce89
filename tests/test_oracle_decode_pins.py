"""Pins of the oracle functions every GPU decode test is compared against,
taken from what the pages and the mathematics fix (not from the oracle):

* QJL decode logits (QJL summary, Definition 3.1 and Lemma 3.2: the
  estimator sqrt(pi/2)/m * ||k|| * <S q, sign(S k)> is unbiased for <q, k>
  when the rows of S are N(0, I)): the mean over 10^4 seeded S of the
  oracle's decode logit of every key lies within 4 standard errors of
  scale * (nu / ||k||) * q.k, nu being the stored binary16 norm. The same for
  the outlier split (QJL "处理异常值（Outliers）": two independent instances,
  each unbiased for its own coordinates), whose expectation is the sum of the
  two instances' inner products. A wrong sqrt(pi/2)/m, a flipped sign
  convention or a wrong outlier-instance factor moves the mean by many
  standard errors. The packed-page path (decode_arena_head) is then shown to
  give the very same logits as the estimator on directly computed bits.
* MixKVQ pages with mixed tiers through dequant_mixkvq_page (MixKVQ
  three-tier scheme; KIVI blog section 2 min-max contract): every channel
  lands at its own position (a random channel order), the BF16 channel is
  exact and every quantized channel is within half a step of the original,
  |k - k^| <= s/2 with s = (max - min)/(2^b - 1) of that channel at its own
  tier (plus the binary16 rounding of the stored step), which a UINT4 channel
  read at two bits, or a channel read from another position, violates.
* PN-Mix pages (PN-Mix "核心公式" Eq.2 and Eq.7, Appendix G planes): the
  unpacked codes equal the 3-bit min-max codes of the high channels and the
  1-bit midpoint codes of the low ones, code for code, and the dequantized
  Keys are within s/2 (3-bit) or (max - min)/4 (1-bit midpoint) of the input.
"""
import math

import numpy as np

from oracle import attention, flush, layout, qjl
from oracle.numerics import bf16_to_f64, f16_to_f64
from oracle.quant import dequantize, quantize_groups, quantize_groups_midpoint

D = 128
SCALE = 1.0 / math.sqrt(D)


def rand_bf16(rng, shape, scale=1.0, shift=0.0):
    x = (rng.standard_normal(shape) * scale + shift).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)   # truncation: still a bf16 pattern


def gaussian_s(rng, rows):
    """i.i.d. N(0, 1) sketch rows (Definition 3.1's S), stored as bf16."""
    return rand_bf16(rng, (rows, D))


def mc_check(mean, sd, n, expect):
    se = sd / math.sqrt(n)
    z = np.abs(mean - expect) / se
    assert np.all(z <= 4.0), (z.max(), int(np.argmax(z)))
    return z


def test_qjl_decode_logits_unbiased():
    rng = np.random.default_rng(2025)
    T, m, N = 32, 256, 10000
    q = rand_bf16(rng, (1, D))
    K = rand_bf16(rng, (T, D))
    q64, K64 = bf16_to_f64(q)[0], bf16_to_f64(K)
    norms = qjl.key_norms(K)
    V = np.zeros((T, D))
    s1 = np.zeros(T)
    s2 = np.zeros(T)
    for _ in range(N):
        S = gaussian_s(rng, m)
        bits = qjl.sketch_bits(S, K)
        _, _, lg = attention.decode_kv_head(q64[None], np.zeros((T, D)), V, SCALE, qjl=(S, bits, norms),
                                            with_logits=True)
        s1 += lg[0]
        s2 += lg[0] ** 2
    mean = s1 / N
    sd = np.sqrt(s2 / N - mean ** 2)
    # the estimator is unbiased for <q, k> with the exact norm; the cache holds
    # nu = binary16(||k||), which scales the expectation by nu / ||k||
    expect = SCALE * (f16_to_f64(norms) / np.linalg.norm(K64, axis=1)) * (K64 @ q64)
    mc_check(mean, sd, N, expect)
    # the band is tight enough to see a flipped sign or a 1/m factor
    assert np.all(np.abs(-expect - mean) > 8 * sd / math.sqrt(N))
    assert np.mean(np.abs(mean * math.sqrt(2 / math.pi) - expect)) > 10 * np.mean(sd / math.sqrt(N))


def test_qjl_split_decode_logits_unbiased():
    rng = np.random.default_rng(2026)
    T, m, mo, N = 32, 256, 64, 10000
    q = rand_bf16(rng, (1, D))
    K = rand_bf16(rng, (T, D))
    outl = np.zeros(D, bool)
    outl[rng.choice(D, 8, replace=False)] = True
    K[:, outl] = rand_bf16(rng, (T, 8), scale=20.0)   # outlier channels carry most of ||k||
    q64, K64 = bf16_to_f64(q)[0], bf16_to_f64(K)
    _, nu_i, nu_o = qjl.split_sketch(gaussian_s(rng, m + mo), m, K, outl)   # the norms do not depend on S
    V = np.zeros((T, D))
    s1 = np.zeros(T)
    s2 = np.zeros(T)
    keep_i = np.where(outl, 0, 0xFFFF).astype(np.uint16)
    keep_o = np.where(outl, 0xFFFF, 0).astype(np.uint16)
    for _ in range(N):
        S = gaussian_s(rng, m + mo)
        # each instance's sign bits: its rows restricted to its own channels
        bits = np.concatenate([qjl.sketch_bits(S[:m] & keep_i, K), qjl.sketch_bits(S[m:] & keep_o, K)])
        _, _, lg = attention.decode_kv_head(q64[None], np.zeros((T, D)), V, SCALE,
                                            qjl=(S, m, outl, bits, nu_i, nu_o), with_logits=True)
        s1 += lg[0]
        s2 += lg[0] ** 2
    mean = s1 / N
    sd = np.sqrt(s2 / N - mean ** 2)
    ki, ko = np.where(outl, 0.0, K64), np.where(outl, K64, 0.0)
    qi, qo = np.where(outl, 0.0, q64), np.where(outl, q64, 0.0)
    expect = SCALE * (f16_to_f64(nu_i) / np.linalg.norm(ki, axis=1) * (ki @ qi)
                      + f16_to_f64(nu_o) / np.linalg.norm(ko, axis=1) * (ko @ qo))
    mc_check(mean, sd, N, expect)
    # an outlier term scaled by 1/m instead of 1/m_o is biased by 3/4 of it
    wrong = expect - 0.75 * SCALE * f16_to_f64(nu_o) / np.linalg.norm(ko, axis=1) * (ko @ qo)
    assert np.max(np.abs(wrong - mean) / (sd / math.sqrt(N))) > 8


def test_qjl_arena_logits_equal_estimator_on_bits():
    """decode_arena_head unpacks the page and gives, bit for bit, the logits
    of the estimator on the sketch computed straight from S and K."""
    rng = np.random.default_rng(7)
    K = rand_bf16(rng, (128, D))
    V = rand_bf16(rng, (128, D))
    q = rand_bf16(rng, (4, D))
    q64 = bf16_to_f64(q)
    S = gaussian_s(rng, 256)
    page = flush.flush_qjl_page(K, V, S)
    _, _, lg_a = attention.decode_arena_head(2, q, [page], SCALE, s_bits=S, with_logits=True)
    _, _, lg_d = attention.decode_kv_head(q64, np.zeros((128, D)), np.zeros((128, D)), SCALE,
                                          qjl=(S, qjl.sketch_bits(S, K), qjl.key_norms(K)), with_logits=True)
    assert np.array_equal(lg_a, lg_d)
    # outlier split through the page
    outl = np.zeros(D, bool)
    outl[rng.choice(D, 8, replace=False)] = True
    S2 = gaussian_s(rng, 256 + 64)
    page2 = flush.flush_qjl_page(K, V, S2, m=256, outl=outl)
    _, _, lg_a2 = attention.decode_arena_head(2, q, [page2], SCALE, s_bits=S2, qjl_m=256, outl=outl,
                                              with_logits=True)
    bits, nu_i, nu_o = qjl.split_sketch(S2, 256, K, outl)
    _, _, lg_d2 = attention.decode_kv_head(q64, np.zeros((128, D)), np.zeros((128, D)), SCALE,
                                           qjl=(S2, 256, outl, bits, nu_i, nu_o), with_logits=True)
    assert np.array_equal(lg_a2, lg_d2)


def _half_step_bound(x64, b):
    """s/2 of a min-max group at b bits, plus the binary16 rounding of the
    stored step (at most 2^-11 relative, times the largest code)."""
    M, mn = x64.max(), x64.min()
    s = (M - mn) / (2 ** b - 1)
    return s / 2 + (2 ** b - 1) * s * 2.0 ** -11 + 1e-12


def test_mixkvq_tiered_page_dequant():
    rng = np.random.default_rng(11)
    for n16, n4 in ((1, 12), (16, 32), (5, 0), (0, 7)):
        K = rand_bf16(rng, (128, D))
        out_ch = rng.choice(D, 8, replace=False)
        K[:, out_ch] = rand_bf16(rng, (128, 8), scale=15.0, shift=5.0)
        V = rand_bf16(rng, (128, D))
        perm = rng.permutation(D).astype(np.uint8)   # not sorted: placement matters
        page = flush.flush_mixkvq_page(K, V, perm, n16, n4)
        Kh, Vh = attention.dequant_mixkvq_page(page, n16, n4, perm)
        K64, V64 = bf16_to_f64(K), bf16_to_f64(V)
        p = perm.astype(np.int64)
        for pos, c in enumerate(p):
            if pos < n16:
                assert np.array_equal(Kh[:, c], K64[:, c]), (n16, n4, c)
                continue
            b = 4 if pos < n16 + n4 else 2
            err = np.abs(Kh[:, c] - K64[:, c]).max()
            assert err <= _half_step_bound(K64[:, c], b), (n16, n4, pos, c, b, err)
            codes, sc, of = quantize_groups(K[:, c][None], b)
            assert np.array_equal(Kh[:, c], dequantize(codes, sc[:, None], of[:, None])[0]), (n16, n4, c)
        # a UINT4 channel read at two bits, or a channel read at another
        # channel's position, breaks the bound somewhere in this page
        if n4:
            c4 = p[n16]
            assert np.abs(Kh[:, c4] - K64[:, c4]).max() < _half_step_bound(K64[:, c4], 4)
        # values: per token, 4 groups of 32 channels, 2 bits
        for t in range(128):
            for j in range(4):
                sl = slice(32 * j, 32 * j + 32)
                assert np.abs(Vh[t, sl] - V64[t, sl]).max() <= _half_step_bound(V64[t, sl], 2)


def test_pnmix_unpack_codes_and_bounds():
    rng = np.random.default_rng(12)
    for layout_name in ("half", "adjacent"):
        pairs = rng.choice(64, 32, replace=False)
        hi = np.zeros(D, bool)
        if layout_name == "half":
            hi[pairs] = True
            hi[pairs + 64] = True
        else:
            hi[2 * pairs] = True
            hi[2 * pairs + 1] = True
        K = rand_bf16(rng, (128, D))
        V = rand_bf16(rng, (128, D))
        page = flush.flush_pnmix_page(K, V, hi)
        u = layout.unpack_pnmix_page(page, hi)
        hi_idx, lo_idx = np.nonzero(hi)[0], np.nonzero(~hi)[0]
        c3, s3, o3 = quantize_groups(K[:, hi_idx].T, 3)
        c1, s1, o1 = quantize_groups_midpoint(K[:, lo_idx].T)
        assert np.array_equal(u["codes"][hi_idx], c3)
        assert np.array_equal(u["codes"][lo_idx], c1)
        assert np.array_equal(u["scale"][hi_idx], s3) and np.array_equal(u["offset"][hi_idx], o3)
        assert np.array_equal(u["scale"][lo_idx], s1) and np.array_equal(u["offset"][lo_idx], o1)
        Kh, _ = attention.dequant_pnmix_page(page, hi)
        K64 = bf16_to_f64(K)
        for c in hi_idx:
            assert np.abs(Kh[:, c] - K64[:, c]).max() <= _half_step_bound(K64[:, c], 3), c
        for c in lo_idx:
            M, mn = K64[:, c].max(), K64[:, c].min()
            # Eq.7: levels (3m+M)/4 and (m+3M)/4, error at most (M-m)/4; the
            # stored z and s are binary16 roundings (2^-11 relative each)
            slack = (abs(3 * mn + M) / 4 + (M - mn) / 2) * 2.0 ** -11 + 1e-12
            assert np.abs(Kh[:, c] - K64[:, c]).max() <= (M - mn) / 4 + slack, c
