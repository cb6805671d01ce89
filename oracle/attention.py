"""Single-token decode attention over the mixed cache (oracle).

The method computes, up to rounding order, the plain dense attention over the
dequantized cache, so the oracle is that definition written out in float64:
s = q K^T * scale, p = softmax(s) over ALL visible tokens, o = p V (KIVI blog
section 1 and section 6: the quantized history and the full-precision
residual share one global softmax, with the Value boundary taken on its own
side). MixKVQ Algorithm 1 (Decoding) sums the per-tier partial dot products
before one softmax. PN-Mix puts the attention-sink tokens and the residual in
full precision next to the packed pages (flowchart, "B[sink 原精度保护与
residual 缓冲]"). QJL replaces q.k of a sketched key by the estimator of
Definition 3.1 (Algorithm 1 steps 4-5).

Readings: the scale is 1/sqrt(head_dim) for every key mode (MixKVQ calls D the
hidden size, a slip; the KIVI blog and the attention formula use the head
dimension); QJL's estimate gets the same 1/sqrt(D) so that its logits are on
the scale of q.k/sqrt(D).
"""
from __future__ import annotations

import math

import numpy as np

from . import layout
from .numerics import bf16_to_f64, f16_to_f64
from .quant import dequantize
from .qjl import estimate_scores, estimate_scores_split
from .select import hi_channels_from_record

D = 128


def dequant_values(vpart) -> np.ndarray:
    codes, scale, offset = vpart
    return dequantize(codes, np.repeat(scale, 32, axis=1), np.repeat(offset, 32, axis=1))


def dequant_mixkvq_page(page, n16, n4, perm):
    u = layout.unpack_mixkvq_page(page, n16, n4, perm)
    perm = np.asarray(perm, dtype=np.int64)
    K = np.zeros((128, D))
    K[:, perm[:n16]] = bf16_to_f64(u["kbf"]).T
    c4, s4, o4 = u["k4"]
    if n4:
        K[:, perm[n16:n16 + n4]] = dequantize(c4, s4[:, None], o4[:, None]).T
    c2, s2, o2 = u["k2"]
    if c2.shape[0]:
        K[:, perm[n16 + n4:]] = dequantize(c2, s2[:, None], o2[:, None]).T
    return K, dequant_values(u["v"])


def dequant_pnmix_page(page, hi_channels):
    u = layout.unpack_pnmix_page(page, hi_channels)
    K = dequantize(u["codes"], u["scale"][:, None], u["offset"][:, None]).T
    return K, dequant_values(u["v"])


def qjl_page_parts(page, m, m_out=0):
    u = layout.unpack_qjl_page(page, m, m_out)
    return u["bits"][:m + m_out], u["norms"], u.get("norms_out"), dequant_values(u["v"])


def softmax_attend(logits: np.ndarray, values: np.ndarray):
    """One global softmax over all logits, then the weighted sum of values."""
    mx = logits.max()
    e = np.exp(logits - mx)
    p = e / e.sum()
    return p @ values, p


def decode_kv_head(q_heads, K_q, V_q, scale, sink=None, resid=None, qjl=None, with_logits=False):
    """Attention of the g query heads of one KV head.

    q_heads [g, D] float64; K_q/V_q [Tq, D] the dequantized page tokens
    (ignored for QJL keys, where ``qjl`` = (S bits, sign bits [m,Tq],
    norm bits [Tq]) supplies the estimator, or with the outlier split
    (S bits, m, outlier channels, sign bits, normal norms, outlier norms));
    sink/resid = (K, V) float64.
    Returns (out [g, D], probs [g, T_total]), and the logits [g, T_total]
    (scale included) with with_logits."""
    segs_k, segs_v, kinds = [], [], []
    if sink is not None and sink[0].shape[0]:
        segs_k.append(sink[0]); segs_v.append(sink[1]); kinds.append("exact")
    if V_q.shape[0]:
        segs_k.append(K_q); segs_v.append(V_q); kinds.append("qjl" if qjl is not None else "exact")
    if resid is not None and resid[0].shape[0]:
        segs_k.append(resid[0]); segs_v.append(resid[1]); kinds.append("exact")
    values = np.concatenate(segs_v, axis=0) if segs_v else np.zeros((0, D))
    outs, probs, logit_rows = [], [], []
    for q in q_heads:
        parts = []
        for kk, kind in zip(segs_k, kinds):
            if kind == "exact":
                parts.append(kk @ q * scale)
            elif len(qjl) == 6:          # QJL outlier split: two instances (outlier paragraph)
                s_bits, m, outl, bits, nu_i, nu_o = qjl
                parts.append(estimate_scores_split(q, s_bits, m, outl, bits, nu_i, nu_o) * scale)
            else:                        # plain QJL, Definition 3.1 / Algorithm 1 EstimateScores
                s_bits, bits, norms = qjl
                parts.append(estimate_scores(q, s_bits, bits, norms) * scale)
        logits = np.concatenate(parts) if parts else np.zeros(0)
        o, p = softmax_attend(logits, values)
        outs.append(o)
        probs.append(p)
        logit_rows.append(logits)
    if with_logits:
        return np.array(outs), np.array(probs), np.array(logit_rows)
    return np.array(outs), np.array(probs)


def kl_divergence(p_ref: np.ndarray, p_q: np.ndarray) -> float:
    """KL(p_ref || p_q), the attention-fidelity number the PN-Mix notes report."""
    mask = p_ref > 0
    return float(np.sum(p_ref[mask] * (np.log(p_ref[mask]) - np.log(p_q[mask]))))


def decode_arena_head(key_mode, q_bits_heads, arena_pages, scale, *, n16=0, n4=0, perm=None,
                      mask_rec=None, pair_layout="half", s_bits=None,
                      sink_k=None, sink_v=None, resid_k=None, resid_v=None, page_perms=None,
                      qjl_m=None, outl=None, with_logits=False, n_vq=None, vwin=None):
    """Decode for one (batch, KV head) from packed pages.

    q_bits_heads [g, D] bf16 bits; arena_pages: list of page byte arrays;
    sink_*/resid_* [n, D] bf16 bits (or None); page_perms: MixKVQ channel
    order of each page (per-flush reselection), else `perm` for every page;
    qjl_m / outl: the QJL outlier split (normal rows, outlier channels).
    n_vq / vwin: KIVI's Value FIFO (KIVI blog sections 4-6): only the Values
    of tokens 0 .. n_vq - 1 are quantized (in the pages); every later token,
    sealed Key page or Key residual alike, takes its Value from the
    full-precision window vwin [T - n_vq, D] (bf16 bits), and resid_v is not
    used. The Key boundary (pages | resid_k) and the Value boundary (n_vq)
    differ; one softmax covers all tokens.
    Returns (out [g, D], probs), and the logits with with_logits."""
    q = bf16_to_f64(q_bits_heads)
    Ks, Vs, bits_l, norms_l, norms_o = [], [], [], [], []
    split = key_mode == 2 and outl is not None
    hi = hi_channels_from_record(mask_rec, pair_layout) if key_mode == 1 else None
    for i, page in enumerate(arena_pages):
        if key_mode == 0:
            K, V = dequant_mixkvq_page(page, n16, n4, perm if page_perms is None else page_perms[i])
        elif key_mode == 1:
            K, V = dequant_pnmix_page(page, hi)
        else:
            m = qjl_m if split else s_bits.shape[0]
            b, nrm, nrm_o, V = qjl_page_parts(page, m, s_bits.shape[0] - m)
            K = np.zeros((128, D))
            bits_l.append(b)
            norms_l.append(nrm)
            norms_o.append(nrm_o)
        Ks.append(K)
        Vs.append(V)
    K_q = np.concatenate(Ks) if Ks else np.zeros((0, D))
    V_q = np.concatenate(Vs) if Vs else np.zeros((0, D))
    qjl = None
    if key_mode == 2 and bits_l:
        qjl = (s_bits, np.concatenate(bits_l, axis=1), np.concatenate(norms_l))
        if split:
            qjl = (s_bits, qjl_m, outl, qjl[1], qjl[2], np.concatenate(norms_o))
    sink = None if sink_k is None else (bf16_to_f64(sink_k), bf16_to_f64(sink_v))
    if vwin is not None:
        W = bf16_to_f64(vwin)
        Tk = V_q.shape[0]
        n_kres = 0 if resid_k is None else resid_k.shape[0]
        assert n_vq <= Tk and W.shape[0] == Tk + n_kres - n_vq
        V_q = V_q.copy()
        V_q[n_vq:] = W[:Tk - n_vq]
        resid = None if resid_k is None else (bf16_to_f64(resid_k), W[Tk - n_vq:])
    else:
        resid = None if resid_k is None else (bf16_to_f64(resid_k), bf16_to_f64(resid_v))
    return decode_kv_head(q, K_q, V_q, scale, sink=sink, resid=resid, qjl=qjl, with_logits=with_logits)


def fifo_page(page, off_v: int, n_rows: int) -> np.ndarray:
    """A page as KIVI's Value FIFO leaves it (KIVI blog section 4): its Keys
    sealed, Values quantized only for its first n_rows tokens (those that
    have left the full-precision window); the other rows hold code 0 and a
    zero scale and offset."""
    page = np.array(page, dtype=np.uint8, copy=True)
    codes, sc, of = layout.unpack_v(page[off_v:])
    codes[n_rows:] = 0
    sc[n_rows:] = 0
    of[n_rows:] = 0
    page[off_v: off_v + layout.V_CODE_BYTES + layout.V_META_BYTES] = layout.pack_v(codes, sc, of)
    return page


def reference_attention(q_bits_heads, k_bits, v_bits, scale):
    """Unquantized attention on the bf16 cache (the fidelity baseline)."""
    q = bf16_to_f64(q_bits_heads)
    K = bf16_to_f64(k_bits)
    V = bf16_to_f64(v_bits)
    outs, probs = [], []
    for qq in q:
        o, p = softmax_attend(K @ qq * scale, V)
        outs.append(o)
        probs.append(p)
    return np.array(outs), np.array(probs)
