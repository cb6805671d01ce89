"""Residual-buffer state machine (oracle).

KIVI blog sections 4-5: a Key goes to the full-precision residual and, once
the residual holds R tokens, the whole segment is quantized, appended to the
quantized history and the residual is cleared, so the persisted Key residual
cycles through 0..R-1 (its mean over a full cycle is (R-1)/2). KIVI's Value
side uses a FIFO of length R instead. The paper's Algorithm 1 appends,
adjusts the cache and then attends; the fixed flash implementation appends
K, forms the logits, seals a full Key segment, appends V, forms the output
and only then moves the oldest Value out.

MixKVQ Algorithm 1 (Decoding) applies the Key rule to both Keys and Values:
append, flush both when the residual reaches R, then attend. This library
follows that rule; the flush is a separate call so the caller picks whether
it attends before or after sealing.
"""
from __future__ import annotations


def kivi_flash_trace(R: int, G: int, steps: int):
    """Token-id bookkeeping of the fixed flash decode order.

    Returns per step (k_compute_full_len, k_persist_full_len,
    v_compute_full_len, v_persist_full_len, k_compute, v_compute)."""
    if G <= 0 or R <= 0 or R % G:
        raise ValueError("positive G and R with R divisible by G required")
    kq, kr, vq, vr = [], [], [], []
    rows = []
    for token in range(1, steps + 1):
        kr.append(token)
        k_compute = (list(kq), list(kr))
        if len(kr) == R:
            kq.extend(kr)
            kr = []
        vr.append(token)
        v_compute = (list(vq), list(vr))
        if len(vr) > R:
            vq.append(vr.pop(0))
        rows.append((len(k_compute[1]), len(kr), len(v_compute[1]), len(vr), k_compute, v_compute))
    return rows


def mixkvq_decode_trace(R: int, steps: int, start_resid: int = 0):
    """Residual length seen by attention and kept after each MixKVQ decode
    step (append, flush at R, attend): returns (attend_len, persist_len)."""
    r = start_resid
    out = []
    for _ in range(steps):
        r += 1
        if r == R:
            r = 0
        out.append((r, r))
    return out
