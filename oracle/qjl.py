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
    """[T] binary16 bit patterns of ||k_t||_2, correctly rounded."""
    out = np.zeros(k_bits.shape[0], dtype=np.uint16)
    for t in range(k_bits.shape[0]):
        s = sum((bf16_fraction(int(b)) ** 2 for b in k_bits[t]), Fraction(0))
        out[t] = rn_f16_sqrt_bits(s)
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
