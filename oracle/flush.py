"""Flush of a full 128-token residual buffer into one packed page (oracle).

MixKVQ page, Algorithm 1 (Decoding, KeyQuant, GroupQuant) and "通过延迟更新
进行摊销调度": once the full-precision buffer holds R tokens the Keys are
quantized per channel over those tokens (G = R = 128 here, one group per
channel per page) with each channel's tier, the Values per token in groups of
32 channels, then everything is packed and merged into the main cache.
KIVI blog section 3 fixes the grouping axes (Key K[t:t+G, d] per channel,
Value V[t, d:d+G] per token). PN-Mix ("核心公式", Appendix G): high channels
at 3 bits, low channels at 1 bit with the midpoint correction. QJL: sign
sketch plus norm (Algorithm 1 steps 2-3).
"""
from __future__ import annotations

import numpy as np

from . import layout
from .qjl import key_norms, sketch_bits, split_sketch
from .quant import quantize_groups, quantize_groups_midpoint

D = 128
G_V = 32


def quantize_values(v_bits: np.ndarray):
    """Per-token 2-bit value quantization in groups of 32 channels.

    v_bits [T][128] -> (codes [T][128], scale [T][4], offset [T][4])."""
    T = v_bits.shape[0]
    groups = v_bits.reshape(T * (D // G_V), G_V)
    codes, scale, offset = quantize_groups(groups, 2)
    return codes.reshape(T, D), scale.reshape(T, D // G_V), offset.reshape(T, D // G_V)


def flush_mixkvq_page(k_bits, v_bits, perm, n16, n4) -> np.ndarray:
    """k_bits, v_bits [128 t][128 ch] bf16 bits -> packed page bytes."""
    n2 = D - n16 - n4
    perm = np.asarray(perm, dtype=np.int64)
    ch4 = perm[n16: n16 + n4]
    ch2 = perm[n16 + n4:]
    k4 = quantize_groups(k_bits[:, ch4].T, 4) if n4 else (np.zeros((0, 128), np.uint8),) + (np.zeros(0, np.uint16),) * 2
    k2 = quantize_groups(k_bits[:, ch2].T, 2) if n2 else (np.zeros((0, 128), np.uint8),) + (np.zeros(0, np.uint16),) * 2
    v = quantize_values(v_bits)
    return layout.pack_mixkvq_page(n16, n4, perm, k_bits, k4, k2, v)


def flush_pnmix_page(k_bits, v_bits, hi_channels) -> np.ndarray:
    hi = np.asarray(hi_channels, dtype=bool)
    codes = np.zeros((D, 128), np.uint8)
    scale = np.zeros(D, np.uint16)
    offset = np.zeros(D, np.uint16)
    hi_idx = np.nonzero(hi)[0]
    lo_idx = np.nonzero(~hi)[0]
    if hi_idx.size:
        c, s, o = quantize_groups(k_bits[:, hi_idx].T, 3)
        codes[hi_idx], scale[hi_idx], offset[hi_idx] = c, s, o
    if lo_idx.size:
        c, s, o = quantize_groups_midpoint(k_bits[:, lo_idx].T)
        codes[lo_idx], scale[lo_idx], offset[lo_idx] = c, s, o
    v = quantize_values(v_bits)
    return layout.pack_pnmix_page(hi, codes, scale, offset, v)


def flush_qjl_page(k_bits, v_bits, s_bits, m=None, outl=None) -> np.ndarray:
    """QJL page of 128 tokens. s_bits [m (+ m_o), D]; with the outlier split
    (outl: [D] bool outlier channels of the head) rows m.. are the outlier
    instance."""
    v = quantize_values(v_bits)
    if outl is None:
        m = s_bits.shape[0]
        return layout.pack_qjl_page(m, sketch_bits(s_bits, k_bits), key_norms(k_bits), v)
    bits, nu_i, nu_o = split_sketch(s_bits, m, k_bits, outl)
    return layout.pack_qjl_page(m, bits, nu_i, v, norms_out=nu_o)
