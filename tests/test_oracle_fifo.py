"""Pins of the oracle's KIVI Value-FIFO decode (KIVI blog sections 4-6): the
Key boundary (sealed pages | Key residual) and the Value boundary (quantized
Values of the oldest tokens | the full-precision window) are separate, and
one softmax covers every token.

* Closed form: with every Key zero the attention is uniform, and with Value
  groups (0, 1.40625, 3, ..., 3) the 2-bit code of channel 1 dequantizes to
  exactly 1, so the output's channel 1 is (n_vq * 1 + (T - n_vq) * 1.40625)/T
  for n_vq quantized Values among T tokens, whatever the page holds for the
  later tokens; an off-by-one in the boundary moves it by 0.40625/T.
* With the Value boundary on the Key boundary (n_vq = every sealed token) the
  FIFO decode is the ordinary decode with the window as the residual Values.
* A FIFO page holds its first n Value rows exactly as the flushed page does
  and zero codes, scales and offsets after them.
"""
import math

import numpy as np

from oracle import attention, flush, layout
from oracle.numerics import bf16_to_f64

D = 128


def bf16(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rand_bf16(rng, shape):
    return bf16(rng.standard_normal(shape))


def test_fifo_boundary_closed_form():
    n_pages, n_kres = 2, 37
    T = 128 * n_pages + n_kres
    K = np.zeros((T, D), np.uint16)                                  # bf16 +0: every logit 0
    row = np.full(D, 3.0, np.float32)
    row[0::32] = 0.0
    row[1::32] = 1.40625                                             # exact in bf16
    V = np.tile(bf16(row), (T, 1))
    perm = np.arange(D, dtype=np.uint8)
    q = bf16(np.ones((4, D)))
    pages = [flush.flush_mixkvq_page(K[128 * p:128 * p + 128], V[128 * p:128 * p + 128], perm, 1, 12)
             for p in range(n_pages)]
    for n_vq in (0, 1, 127, 128, 200, 256):
        out, probs = attention.decode_arena_head(0, q, pages, 1 / math.sqrt(D), n16=1, n4=12, perm=perm,
                                                 resid_k=K[128 * n_pages:], n_vq=n_vq, vwin=V[n_vq:])
        assert np.allclose(probs, 1.0 / T, rtol=0, atol=1e-15)
        want = (n_vq * 1.0 + (T - n_vq) * 1.40625) / T
        assert abs(out[0, 1] - want) < 1e-12, (n_vq, out[0, 1], want)
        assert abs(out[0, 0]) < 1e-12 and abs(out[0, 2] - 3.0) < 1e-12
    # the same with FIFO pages (later Value rows zero): nothing changes
    off_v = layout.mixkvq_geometry(1, 12)["off_v"]
    n_vq = 200
    fp = [attention.fifo_page(pages[0], off_v, 128), attention.fifo_page(pages[1], off_v, n_vq - 128)]
    out2, _ = attention.decode_arena_head(0, q, fp, 1 / math.sqrt(D), n16=1, n4=12, perm=perm,
                                          resid_k=K[128 * n_pages:], n_vq=n_vq, vwin=V[n_vq:])
    assert abs(out2[0, 1] - (n_vq + (T - n_vq) * 1.40625) / T) < 1e-12


def test_fifo_on_key_boundary_is_ordinary_decode():
    rng = np.random.default_rng(4)
    n_pages, n_kres = 3, 50
    T = 128 * n_pages + n_kres
    K, V = rand_bf16(rng, (T, D)), rand_bf16(rng, (T, D))
    q = rand_bf16(rng, (4, D))
    perm = rng.permutation(D).astype(np.uint8)
    pages = [flush.flush_mixkvq_page(K[128 * p:128 * p + 128], V[128 * p:128 * p + 128], perm, 1, 12)
             for p in range(n_pages)]
    Tk = 128 * n_pages
    a, pa = attention.decode_arena_head(0, q, pages, 0.09, n16=1, n4=12, perm=perm, resid_k=K[Tk:], n_vq=Tk,
                                        vwin=V[Tk:])
    b, pb = attention.decode_arena_head(0, q, pages, 0.09, n16=1, n4=12, perm=perm, resid_k=K[Tk:],
                                        resid_v=V[Tk:])
    assert np.array_equal(a, b) and np.array_equal(pa, pb)
    # moving the Value boundary back swaps quantized Values for exact ones, token by token
    c, _ = attention.decode_arena_head(0, q, pages, 0.09, n16=1, n4=12, perm=perm, resid_k=K[Tk:], n_vq=Tk - 5,
                                       vwin=V[Tk - 5:])
    Kq = np.concatenate([attention.dequant_mixkvq_page(p, 1, 12, perm)[0] for p in pages])
    Vq = np.concatenate([attention.dequant_mixkvq_page(p, 1, 12, perm)[1] for p in pages])
    Vmix = np.concatenate([Vq[:Tk - 5], bf16_to_f64(V[Tk - 5:])])
    Kall = np.concatenate([Kq, bf16_to_f64(K[Tk:])])
    for h in range(4):
        ref, _ = attention.softmax_attend(Kall @ bf16_to_f64(q[h]) * 0.09, Vmix)
        assert np.allclose(c[h], ref, rtol=0, atol=1e-12)


def test_fifo_page_rows():
    rng = np.random.default_rng(5)
    K, V = rand_bf16(rng, (128, D)), rand_bf16(rng, (128, D))
    page = flush.flush_mixkvq_page(K, V, np.arange(D, dtype=np.uint8), 1, 12)
    off_v = layout.mixkvq_geometry(1, 12)["off_v"]
    for n in (0, 1, 37, 127, 128):
        fp = attention.fifo_page(page, off_v, n)
        assert np.array_equal(fp[:off_v], page[:off_v])            # Keys untouched
        c0, s0, o0 = layout.unpack_v(page[off_v:])
        c1, s1, o1 = layout.unpack_v(fp[off_v:])
        assert np.array_equal(c1[:n], c0[:n]) and np.array_equal(s1[:n], s0[:n]) and np.array_equal(o1[:n], o0[:n])
        assert not c1[n:].any() and not s1[n:].any() and not o1[n:].any()
