"""Residual-buffer bookkeeping (oracle).

KIVI blog sections 4-5. Keys are grouped along time: a Key stays in the
full-precision residual until R of them have gathered, then the whole segment
is quantized and the residual starts again, so after t tokens the persisted
Key residual holds t mod R tokens (mean (R - 1)/2 over a full cycle). Values
are grouped along channels, so they can leave the residual one at a time: the
Value residual is a first-in first-out window of the last R tokens, and after
t tokens it holds min(t, R) of them.

Section 5 separates what one decode step computes with from what it leaves
behind: the step attends with the new token already in both residuals, the
Key segment is sealed after the logits are formed, and the oldest Value
leaves the window after the output is formed. So at step t the attention sees
a Key residual of t - R * floor((t - 1) / R) tokens (1..R, never 0) and a
Value residual of min(t, R + 1) tokens.

MixKVQ Algorithm 1 (Decoding) applies the Key rule to Keys and Values alike
(append, flush both when the residual reaches R, then attend). The library's
pages follow that rule; the flush is a separate call, so the caller chooses
whether a step attends before or after sealing.
"""
from __future__ import annotations

from typing import NamedTuple, Tuple


class FlashStep(NamedTuple):
    """State at decode step t (1-based) of the section 5 order: residual
    lengths at compute time and after the step, and the token ids (1-based)
    that the step reads as (quantized, full precision) for Keys and Values."""
    k_compute_full: int
    k_persist_full: int
    v_compute_full: int
    v_persist_full: int
    k_split: Tuple[range, range]
    v_split: Tuple[range, range]


def flash_step(R: int, t: int) -> FlashStep:
    """Closed-form state of step t: Keys quantized in whole segments of R,
    Values through a window of R."""
    sealed = R * ((t - 1) // R)          # Key tokens quantized before step t's logits
    k_comp = t - sealed                  # 1..R
    v_comp = min(t, R + 1)               # the window plus the token just appended
    return FlashStep(k_comp, t % R, v_comp, min(t, R),
                     (range(1, sealed + 1), range(sealed + 1, t + 1)),
                     (range(1, t - v_comp + 1), range(t - v_comp + 1, t + 1)))


def kivi_flash_trace(R: int, G: int, steps: int):
    """flash_step for t = 1..steps. G is the quantization group along time;
    a sealed segment of R Keys must split into whole groups."""
    if R < 1 or G < 1 or R % G != 0:
        raise ValueError(f"residual length R={R} must be a positive multiple of the group size G={G}")
    return [flash_step(R, t) for t in range(1, steps + 1)]


def mixkvq_decode_trace(R: int, steps: int, start_resid: int = 0):
    """Residual length seen by attention and kept after each MixKVQ decode
    step (append, flush at R, attend): returns (attend_len, persist_len)."""
    out = []
    for s in range(1, steps + 1):
        r = (start_resid + s) % R
        out.append((r, r))
    return out
