"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module holds input recipes only: tensor shapes, seeds and value
distributions. It contains none of the quantization, selection or attention
arithmetic; both the HIP path and the CPU oracle receive the tensors it makes.

The workloads stand in for the model activations the pages evaluate on
(Llama-3.1-8B and Qwen-32B GQA attention layers, MixKVQ page "实验环境"; QJL
page "实验环境"; PN-Mix page "本地复现"): post-RoPE Q/K/V drawn i.i.d. from
N(0, 1) in float32 and rounded to bfloat16 (round-to-nearest-even, done by
torch), with eight fixed outlier Key channels per KV head for the MixKVQ
workloads (the Key-channel outliers of MixKVQ page "背景知识与关键观察").
For four of those eight channels the query is attenuated by x0.05 in every
query head of the group, so that a large-range Key channel meets a small
query (the case MixKVQ's query-aware saliency is built for).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

MIXKVQ, PNMIX, QJL = 0, 1, 2
HEAD_DIM = 128
PAGE_TOKENS = 128

# tensor ids folded into the seed so that each tensor is an independent stream
T_QPRE, T_KPRE, T_VPRE, T_QDEC, T_KNEW, T_VNEW, T_SJL, T_OUTL = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    key_mode: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    n_pages: int            # quantized 128-token pages per (batch, kv head)
    n_resid: int            # BF16 residual tokens visible at the decode step
    n_sink: int             # BF16 attention-sink tokens (PN-Mix only)
    seed: int
    n_bf16: int = 0         # MixKVQ tier counts (rest are UINT2)
    n_u4: int = 0
    outlier_scale: float = 0.0   # K outlier channel = scale*z + shift
    outlier_shift: float = 0.0
    n_hi_pairs: int = 32    # PN-Mix: floor(r * D / 2)
    qjl_m: int = 256
    n_append: int = 0       # extra tokens appended after the decode step (C1)
    qjl_outliers: int = 0   # QJL outlier split: outlier channels per (batch, kv head)
    qjl_m_out: int = 0      # ... and the outlier instance's sketch rows

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def prefill_tokens(self) -> int:
        return self.n_sink + self.n_pages * PAGE_TOKENS + self.n_resid

    @property
    def has_outliers(self) -> bool:
        return self.outlier_scale != 0.0

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny MixKVQ: 8 pages + 64 residual, tiers 16/32/80, one decode + one flush
    "tiny_mixkvq": Workload("tiny_mixkvq", MIXKVQ, 1, 4, 1, 8, 64, 0, 1001,
                            n_bf16=16, n_u4=32, outlier_scale=15.0, outlier_shift=5.0,
                            n_append=64),
    # Llama-3.1-8B-shaped layer: 32/8 heads, batch 8, 8192 + 128 residual
    "llama8b_8k": Workload("llama8b_8k", MIXKVQ, 8, 32, 8, 64, 128, 0, 1002,
                           n_bf16=1, n_u4=12, outlier_scale=15.0, outlier_shift=5.0),
    # Qwen-32B-shaped layer: 64/8 heads, batch 16, 32768 context, no residual
    "qwen32b_32k": Workload("qwen32b_32k", MIXKVQ, 16, 64, 8, 256, 0, 0, 1003,
                            n_bf16=1, n_u4=12, outlier_scale=20.0, outlier_shift=0.0),
    # PN-Mix H3/L1: 32/8 heads, batch 32, 32 sink + 16384 + 128 residual
    "pnmix_16k": Workload("pnmix_16k", PNMIX, 32, 32, 8, 128, 128, 32, 1004),
    # QJL: 32/8 heads, batch 64, 32768 context, m = 256
    "qjl_32k": Workload("qjl_32k", QJL, 64, 32, 8, 256, 0, 0, 1005),
    # QJL with the outlier split: the same shape, eight fixed outlier Key
    # channels (20 z) found at the prompt, 64 more sketch rows for them
    "qjl_outlier_32k": Workload("qjl_outlier_32k", QJL, 64, 32, 8, 256, 0, 0, 1006,
                                outlier_scale=20.0, qjl_outliers=8, qjl_m_out=64),
}


def _gen(seed: int, tid: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + tid * 7919) & 0x7FFFFFFFFFFFFFFF)
    return g


def outlier_channels(w: Workload) -> np.ndarray:
    """[batch, n_kv_heads, 8] distinct outlier channel indices; the first four
    of each row are the ones whose query is attenuated."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, T_OUTL])))
    out = np.empty((w.batch, w.n_kv_heads, 8), dtype=np.int64)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            out[b, h] = rng.choice(HEAD_DIM, size=8, replace=False)
    return out


def _apply_k_outliers(k: torch.Tensor, w: Workload, oc: np.ndarray) -> torch.Tensor:
    if not w.has_outliers:
        return k
    idx = torch.as_tensor(oc, device=k.device)                     # [B, Hkv, 8]
    gather = idx[:, :, None, :].expand(-1, -1, k.shape[2], -1)     # [B, Hkv, T, 8]
    vals = torch.gather(k, 3, gather) * w.outlier_scale + w.outlier_shift
    return k.scatter(3, gather, vals)


def _apply_q_attenuation(q: torch.Tensor, w: Workload, oc: np.ndarray) -> torch.Tensor:
    if not w.has_outliers:
        return q
    g = w.group
    idx = torch.as_tensor(oc[:, :, :4], device=q.device)           # [B, Hkv, 4]
    idx = idx.repeat_interleave(g, dim=1)                          # [B, Hq, 4]
    gather = idx[:, :, None, :].expand(-1, -1, q.shape[2], -1)
    vals = torch.gather(q, 3, gather) * 0.05
    return q.scatter(3, gather, vals)


def _normal(shape, seed, tid, device) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, tid, device), device=device, dtype=torch.float32)


def prefill(w: Workload, device="cpu", l_q: Optional[int] = None):
    """Post-RoPE prefill tensors, bf16: q [B,Hq,Lq,D], k and v [B,Hkv,L,D].

    L = sinks + quantized pages + residual; Lq defaults to L (every prefill
    position issues a query)."""
    L = w.prefill_tokens
    l_q = L if l_q is None else l_q
    oc = outlier_channels(w)
    q = _normal((w.batch, w.n_q_heads, l_q, HEAD_DIM), w.seed, T_QPRE, device)
    k = _normal((w.batch, w.n_kv_heads, L, HEAD_DIM), w.seed, T_KPRE, device)
    v = _normal((w.batch, w.n_kv_heads, L, HEAD_DIM), w.seed, T_VPRE, device)
    q = _apply_q_attenuation(q, w, oc)
    k = _apply_k_outliers(k, w, oc)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def decode_query(w: Workload, device="cpu", step: int = 0) -> torch.Tensor:
    """Single-token decode query, bf16 [B, Hq, D]."""
    oc = outlier_channels(w)
    q = _normal((w.batch, w.n_q_heads, 1, HEAD_DIM), w.seed + 7 * step, T_QDEC, device)
    return _apply_q_attenuation(q, w, oc)[:, :, 0, :].to(torch.bfloat16)


def appended_kv(w: Workload, n: int, device="cpu"):
    """n new decode-time K/V tokens per (batch, kv head), bf16 [B, Hkv, n, D]."""
    oc = outlier_channels(w)
    k = _normal((w.batch, w.n_kv_heads, n, HEAD_DIM), w.seed, T_KNEW, device)
    v = _normal((w.batch, w.n_kv_heads, n, HEAD_DIM), w.seed, T_VNEW, device)
    return _apply_k_outliers(k, w, oc).to(torch.bfloat16), v.to(torch.bfloat16)


def qjl_matrix(w: Workload, device="cpu") -> torch.Tensor:
    """The QJL sketch matrix S, bf16 [m (+ m_out), D].

    i.i.d. N(0,1) rows; each block of D rows is orthogonalised by a QR
    factorisation and every row is then rescaled to the length of an
    independent N(0, I_D) draw, so that rows stay marginally Gaussian (QJL
    page "正交化JL变换", which cites orthogonal random features)."""
    m = w.qjl_m
    gen = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, T_SJL])))
    blocks = []
    for _ in range((m + HEAD_DIM - 1) // HEAD_DIM):
        a = gen.standard_normal((HEAD_DIM, HEAD_DIM))
        qmat, rmat = np.linalg.qr(a)
        qmat = qmat * np.sign(np.diag(rmat))[None, :]
        lengths = np.linalg.norm(gen.standard_normal((HEAD_DIM, HEAD_DIM)), axis=1)
        blocks.append(qmat.T * lengths[:, None])
    rows = np.concatenate(blocks, axis=0)[:m]
    if w.qjl_m_out:
        # the outlier instance: i.i.d. N(0,1) rows, used at each head's own
        # outlier columns only (no orthogonalisation over a per-head subset)
        rows = np.concatenate([rows, gen.standard_normal((w.qjl_m_out, HEAD_DIM))], axis=0)
    s = np.ascontiguousarray(rows, dtype=np.float32)
    return torch.from_numpy(s).to(torch.bfloat16).contiguous().to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as raw uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
