"""Pins of the oracle's decode attention.

* KIVI blog section 6: one global softmax over history + residual, the
  117/17 example (and the wrong separate-softmax answer 13.5);
* a cache whose every Key channel is BF16 reduces to plain attention on the
  original bf16 values (MixKVQ's BF16 tier is stored unquantized);
* zero pages reduce to plain attention over the residual / sinks;
* the attention output is invariant to the order of tokens;
* the KIVI blog section 1 error decomposition o^ - o = (p^ - p)V + p^ E_V.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import attention, flush
from oracle.numerics import bf16_to_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_global_softmax_example():
    with open(os.path.join(GOLD, "kivi_global_softmax.json")) as f:
        g = json.load(f)
    nk, nr = g["key_history_len"], g["key_residual_len"]
    logits = np.array([0.0] * nk + [math.log(9)] * nr)
    values = np.array([[float(t), -float(t)] for t in range(1, nk + nr + 1)])
    out, p = attention.softmax_attend(logits, values)
    assert abs(out[0] - float(Fraction(g["out_dim0"]))) < 1e-12
    assert np.allclose(p[:nk], float(Fraction(g["prob_history_each"])), atol=1e-15)
    assert abs(p[-1] - float(Fraction(g["prob_residual"]))) < 1e-15
    # the Value boundary (4 + 5) differs from the Key boundary (8 + 1); splitting
    # p at the Value boundary gives the same output as the dense weighted sum
    vb = g["value_history_len"]
    split = p[:vb] @ values[:vb] + p[vb:] @ values[vb:]
    assert np.allclose(split, out, atol=1e-12)
    # separate softmaxes are wrong: mass 2 and 13.5
    _, p1 = attention.softmax_attend(logits[:nk], values[:nk])
    _, p2 = attention.softmax_attend(logits[nk:], values[nk:])
    wrong = np.concatenate([p1, p2]) @ values
    assert abs(np.concatenate([p1, p2]).sum() - g["wrong_separate_softmax_mass"]) < 1e-12
    assert abs(wrong[0] - float(Fraction(g["wrong_separate_softmax_out_dim0"]))) < 1e-12


def test_all_bf16_tier_is_plain_attention():
    rng = np.random.default_rng(1)
    n_pages, g = 3, 4
    K = rand_bf16(rng, (128 * n_pages, 128))
    V = rand_bf16(rng, (128 * n_pages, 128))
    q = rand_bf16(rng, (g, 128))
    perm = np.arange(128)
    pages = [flush.flush_mixkvq_page(K[128 * p:128 * p + 128], V[128 * p:128 * p + 128], perm, 128, 0)
             for p in range(n_pages)]
    out, probs = attention.decode_arena_head(0, q, pages, 1 / math.sqrt(128), n16=128, n4=0, perm=perm)
    # the Values are still 2-bit quantized: compare against attention with
    # exact keys and the dequantized values
    Vq = np.concatenate([attention.dequant_mixkvq_page(pg, 128, 0, perm)[1] for pg in pages])
    ref_out, ref_p = [], []
    for qq in bf16_to_f64(q):
        o, p = attention.softmax_attend(bf16_to_f64(K) @ qq / math.sqrt(128), Vq)
        ref_out.append(o)
        ref_p.append(p)
    assert np.allclose(out, np.array(ref_out), atol=1e-12, rtol=1e-12)
    assert np.allclose(probs, np.array(ref_p), atol=1e-15)


def test_no_pages_reduces_to_residual_attention():
    rng = np.random.default_rng(2)
    q = rand_bf16(rng, (4, 128))
    rk, rv = rand_bf16(rng, (77, 128)), rand_bf16(rng, (77, 128))
    sk, sv = rand_bf16(rng, (32, 128)), rand_bf16(rng, (32, 128))
    out, _ = attention.decode_arena_head(1, q, [], 0.1, mask_rec=np.zeros(8, np.uint8),
                                         sink_k=sk, sink_v=sv, resid_k=rk, resid_v=rv)
    ref, _ = attention.reference_attention(q, np.concatenate([sk, rk]), np.concatenate([sv, rv]), 0.1)
    assert np.allclose(out, ref, atol=1e-13)


def test_token_order_invariance_and_error_decomposition():
    rng = np.random.default_rng(3)
    T = 300
    K = bf16_to_f64(rand_bf16(rng, (T, 128)))
    V = bf16_to_f64(rand_bf16(rng, (T, 128)))
    q = bf16_to_f64(rand_bf16(rng, (2, 128)))
    perm = rng.permutation(T)
    o1, p1 = attention.decode_kv_head(q, K, V, 0.09)
    o2, _ = attention.decode_kv_head(q, K[perm], V[perm], 0.09)
    assert np.allclose(o1, o2, atol=1e-13)
    # o^ - o = (p^ - p) V + p^ E_V
    EK = rng.standard_normal(K.shape) * 0.01
    EV = rng.standard_normal(V.shape) * 0.01
    oh, ph = attention.decode_kv_head(q, K + EK, V + EV, 0.09)
    lhs = oh - o1
    rhs = (ph - p1) @ V + ph @ EV
    assert np.allclose(lhs, rhs, atol=1e-12)


def test_kl_divergence_basic():
    p = np.array([0.5, 0.5])
    assert attention.kl_divergence(p, p) == 0.0
    assert abs(attention.kl_divergence(p, np.array([0.25, 0.75])) - (0.5 * math.log(2) + 0.5 * math.log(2 / 3))) < 1e-15
