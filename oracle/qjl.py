"""QJL key sketch (oracle).

QJL page, Definition 3.1 and Algorithm 1 ("基于QJL的Key缓存量化算法"):
H_S(k) = sign(S k) with S in R^{m x d}; the cache keeps the m sign bits and
nu = ||k||_2 for every key; the score estimate for a query q is
sqrt(pi/2)/m * nu_j * <S q, sign(S k_j)> and the attention weights are the
softmax of those estimates. The value cache is quantized per token as usual
("Value缓存量化"), which here is the shared 2-bit, 32-channel value codec.

Readings fixed here:
* a sign bit is 1 when S_i . k >= 0 (sign(0) = +1), decided on the EXACT dot
  product of the bf16 rows (the pages are silent on zero);
* nu is stored as binary16, the correctly rounded value of the exact norm;
* S itself is an input (generated on the host, rows orthogonalised as the
  "正交化JL变换" paragraph describes), not computed by the method.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

from .numerics import bf16_fraction, bf16_to_f64, f16_to_f64, rn_f16_sqrt_bits

_U = 2.0 ** -53


def sketch_bits(s_bits: np.ndarray, k_bits: np.ndarray) -> np.ndarray:
    """[m, T] uint8: 1 where the exact S_i . k_t >= 0."""
    S = bf16_to_f64(s_bits)
    K = bf16_to_f64(k_bits)
    dots = S @ K.T                                  # products exact, sum rounded
    mags = np.abs(S) @ np.abs(K).T
    n = S.shape[1]
    gamma = n * _U / (1 - n * _U)
    sure = np.abs(dots) > 2.0 * gamma * mags
    out = (dots >= 0).astype(np.uint8)
    for i, t in zip(*np.nonzero(~sure)):
        exact = sum((bf16_fraction(int(a)) * bf16_fraction(int(b))
                     for a, b in zip(s_bits[i], k_bits[t])), Fraction(0))
        out[i, t] = 1 if exact >= 0 else 0
    return out


def key_norms(k_bits: np.ndarray) -> np.ndarray:
    """[T] binary16 bit patterns of ||k_t||_2, correctly rounded from the
    exact sum of squares. A bf16 value is an integer significand s (< 256)
    times 2^e, so its square is s^2 * 2^(2e): squares sharing an exponent add
    exactly as integers, and the per-exponent sums are joined exactly with
    Python integers on the smallest exponent of the row."""
    b = np.asarray(k_bits, dtype=np.int64)
    if np.any(((b >> 7) & 0xFF) == 0xFF):
        raise ValueError("non-finite bf16")
    e = (b >> 7) & 0xFF
    sig = np.where(e > 0, (b & 0x7F) | 0x80, b & 0x7F)
    ex2 = 2 * (np.maximum(e, 1) - 134)                 # value^2 = sig^2 * 2^ex2
    sq = sig * sig
    out = np.zeros(b.shape[0], dtype=np.uint16)
    for t in range(b.shape[0]):
        nz = sq[t] != 0
        if not nz.any():
            continue
        lo = int(ex2[t][nz].min())
        total = 0
        for u in np.unique(ex2[t][nz]):
            total += int(sq[t][nz & (ex2[t] == u)].sum()) << (int(u) - lo)
        out[t] = rn_f16_sqrt_bits(Fraction(total) * Fraction(2) ** lo)
    return out


def estimate_scores(q_f64: np.ndarray, s_bits: np.ndarray, bits: np.ndarray, norm_bits: np.ndarray) -> np.ndarray:
    """sqrt(pi/2)/m * nu_j * <S q, sign(S k_j)> for every cached key j.

    q_f64 [d]; bits [m, T] (1 = +1, 0 = -1); norm_bits [T] binary16."""
    S = bf16_to_f64(s_bits)
    m = S.shape[0]
    sq = S @ q_f64
    signs = 2.0 * bits.astype(np.float64) - 1.0
    return math.sqrt(math.pi / 2) / m * f16_to_f64(norm_bits) * (sq @ signs)


def prod_qjl(q: np.ndarray, k: np.ndarray, S: np.ndarray) -> float:
    """The estimator of Definition 3.1 on float64 inputs (for statistics)."""
    m = S.shape[0]
    return math.sqrt(math.pi / 2) / m * np.linalg.norm(k) * float((S @ q) @ np.where(S @ k >= 0, 1.0, -1.0))


# --------------------------------------------------------------- outlier split
# QJL page, "处理异常值（Outliers）" with Figure 2: a few fixed Key channels
# carry most of the magnitude; they are found at the prompt phase and the
# outlier and normal parts of every key get two independent QJL instances,
# the outlier one at a lower compression rate (more sketch rows per
# coordinate). Readings fixed here:
# * outlier channels of a (batch, kv head): the n_o largest sums over the
#   prompt's Key tokens of |K_{t,d}| (Figure 2 orders channels by their mean
#   magnitude over tokens), ties to the lower channel; the sums are exact on
#   the psi grid the MixKVQ selection uses;
# * the normal instance is the first m rows of S applied to the normal
#   coordinates k_I (S restricted to those columns); the outlier instance is
#   m_o further i.i.d. N(0,1) rows applied to the outlier coordinates k_O;
# * the score estimate is the sum of the two instances' estimators, each
#   with its own norm (nu_I = ||k_I||, nu_O = ||k_O||, binary16) and its own
#   sqrt(pi/2)/m factor.


def outlier_mask(k_bits: np.ndarray, n_out: int) -> np.ndarray:
    """[D] bool: the n_out channels with the largest exact sum of |K| over
    the prompt's Key tokens k_bits [L, D] (ties: lower channel first)."""
    from .select import psi_sum
    k = np.abs(bf16_to_f64(k_bits)).reshape(-1, k_bits.shape[-1])
    sums = [int(s) for s in psi_sum(k, axis=0)]
    order = sorted(range(len(sums)), key=lambda d: (-sums[d], d))
    out = np.zeros(len(sums), dtype=bool)
    out[order[:n_out]] = True
    return out


def outlier_record(outl: np.ndarray) -> np.ndarray:
    """16-byte record: bit d % 8 of byte d // 8 set for outlier channel d."""
    rec = np.zeros(16, dtype=np.uint8)
    for d in np.nonzero(outl)[0]:
        rec[d // 8] |= np.uint8(1 << (d % 8))
    return rec


def outlier_mask_from_record(rec) -> np.ndarray:
    rec = np.asarray(rec, dtype=np.uint8)
    return np.array([(rec[d // 8] >> (d % 8)) & 1 for d in range(8 * len(rec[:16]))], dtype=bool)


def _restrict(bits: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """bf16 bit rows with the columns outside `keep` set to +0: a dot product
    with such a row is the dot product over the kept coordinates."""
    out = np.array(bits, dtype=np.uint16, copy=True)
    out[..., ~keep] = 0
    return out


def split_sketch(s_bits: np.ndarray, m: int, k_bits: np.ndarray, outl: np.ndarray):
    """The two instances' sign bits and norms of keys k_bits [T, D].

    Returns (bits [m + m_o, T], nu_I [T], nu_O [T]): rows < m are
    sign(S_i . k_I), rows >= m are sign(S_i . k_O)."""
    inl = ~outl
    bits_i = sketch_bits(_restrict(s_bits[:m], inl), k_bits)
    bits_o = sketch_bits(_restrict(s_bits[m:], outl), k_bits)
    nu_i = key_norms(_restrict(k_bits, inl))
    nu_o = key_norms(_restrict(k_bits, outl))
    return np.concatenate([bits_i, bits_o], axis=0), nu_i, nu_o


def estimate_scores_split(q_f64, s_bits, m, outl, bits, nu_i_bits, nu_o_bits) -> np.ndarray:
    """sqrt(pi/2)/m nu_I <S_I q_I, s_I> + sqrt(pi/2)/m_o nu_O <S_O q_O, s_O>."""
    S = bf16_to_f64(s_bits)
    m_o = S.shape[0] - m
    q_i = np.where(outl, 0.0, q_f64)
    q_o = np.where(outl, q_f64, 0.0)
    signs = 2.0 * bits.astype(np.float64) - 1.0
    est_i = math.sqrt(math.pi / 2) / m * f16_to_f64(nu_i_bits) * ((S[:m] @ q_i) @ signs[:m])
    est_o = math.sqrt(math.pi / 2) / m_o * f16_to_f64(nu_o_bits) * ((S[m:] @ q_o) @ signs[m:])
    return est_i + est_o


def prod_qjl_split(q: np.ndarray, k: np.ndarray, S_i: np.ndarray, S_o: np.ndarray, outl: np.ndarray) -> float:
    """The split estimator on float64 inputs (for statistics): the normal
    instance S_i [m, d] and the outlier instance S_o [m_o, d], each applied
    to its own coordinates of q and k."""
    q_i, q_o = np.where(outl, 0.0, q), np.where(outl, q, 0.0)
    k_i, k_o = np.where(outl, 0.0, k), np.where(outl, k, 0.0)
    return prod_qjl(q_i, k_i, S_i) + prod_qjl(q_o, k_o, S_o)
