"""MixKVQ threshold tiers on the GPU (the three-tier rule with tau_BF16 and
tau_UINT4): selection records bit-exact against the oracle, pages laid out by
each head's own tier counts bit-exact, decode (pipelined and generic kernels)
within the decode bound, including thresholds placed exactly on a channel's
salience (the comparisons are strict on the upper side) and capacities that
overflow (the best channels of a full tier stay, the rest move down one).
"""
import math

import numpy as np
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import Pipeline, rel_err
from oracle import attention as oatt
from oracle import flush as oflush
from oracle import select as osel

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

TOL = 2e-3


def salience_quantiles(w, qs):
    """Thresholds at quantiles of A_d over every (batch, kv head) of the
    workload's prefill (computed by the oracle on the host)."""
    q, k, _ = synth.prefill(w, "cpu")
    g = w.group
    vals = []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            qb = synth.bf16_bits(q[b, h * g:(h + 1) * g])
            kb = synth.bf16_bits(k[b, h, w.n_sink:w.n_sink + w.n_pages * 128])
            vals += [float(a) for a in osel.mixkvq_salience(qb, kb)]
    return [float(np.quantile(vals, x)) for x in qs]


CASES = [
    # (workload, its reshaping, quantiles of tau_bf16 / tau_u4, capacities, what the counts show)
    ("llama8b_8k", dict(batch=2, n_kv_heads=4, n_q_heads=16, n_pages=3, n_resid=40), (0.93, 0.7), (32, 64), "varied"),
    # about 13 BF16 and 51 UINT4 candidates per head: both capacities overflow
    ("llama8b_8k", dict(batch=2, n_kv_heads=4, n_q_heads=16, n_pages=3, n_resid=40), (0.9, 0.5), (4, 8), "full"),
    ("qwen32b_32k", dict(batch=2, n_kv_heads=2, n_q_heads=16, n_pages=2, n_resid=0), (0.97, 0.8), (8, 40), "varied"),
    ("tiny_mixkvq", dict(), (0.5, 0.6), (128, 0), "no_u4"),   # tau_bf16 < tau_u4: no UINT4 tier
]


@pytest.mark.parametrize("name,shape,quant,caps,expect", CASES)
def test_threshold_records_pages_decode(name, shape, quant, caps, expect):
    base = synth.WORKLOADS[name]
    w = base.scaled(n_bf16=caps[0], n_u4=caps[1], seed=base.seed + 300, **shape)
    tau = tuple(salience_quantiles(w, quant))
    print(f"\n[case] threshold {w} tau={tau}", flush=True)
    p = Pipeline(w, tau=tau)
    p.select()
    p.flush_prefill()
    p.decode()
    torch.cuda.synchronize()
    fast = p.out.clone()
    p.decode(generic=True)
    torch.cuda.synchronize()
    generic = p.out.clone()
    assert int(p.flags[0].item()) == 0
    counts = set()
    g = p.g
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            rec = p.oracle_record(b, h)
            assert np.array_equal(p.gpu_record(b, h), rec), (b, h)
            counts.add(osel.record_counts(rec))
            pages = [p.oracle_page(b, h, pg, rec) for pg in range(w.n_pages)]
            for pg, ref in enumerate(pages):
                assert p.same_page(p.gpu_page(b, h, pg), ref), (b, h, pg)
            ref_out, _ = p.oracle_decode(b, h, pages, rec)
            for tag, out in (("fast", fast), ("generic", generic)):
                err = rel_err(out.cpu().numpy()[b, h * g:(h + 1) * g], ref_out)
                assert np.all(err <= TOL), (tag, b, h, err)
    print(f"[threshold] {name}: tier counts (BF16, UINT4) per head: {sorted(counts)}")
    if expect == "no_u4":
        assert all(n4 == 0 for _, n4 in counts)
    elif expect == "full":
        assert counts == {caps}
    else:
        assert len(counts) > 1   # the heads' counts differ: per-head page layouts are exercised


def test_threshold_exact_ties():
    """A_d = (d + 1)/48 exactly (every |q| = 1, Key range (d + 1)/16): with
    tau_bf16 = 2.5 and tau_u4 = 2 the channel whose salience equals a
    threshold goes to the lower tier; the page and the decode follow the
    head's counts (8 BF16, 24 UINT4)."""
    dev = "cuda"
    g, lq = 2, 4
    q = torch.ones(1, g, lq, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 1, 128, 128, dtype=torch.float32)
    k[0, 0, 1] = (torch.arange(128, dtype=torch.float32) + 1) / 16
    gen = torch.Generator().manual_seed(5)
    k[0, 0, 2:] = (torch.randn(126, 128, generator=gen).abs() * 0.01).clamp(max=0.05)   # inside [0, 1/16]: ranges unchanged
    k = k.to(torch.bfloat16).to(dev)
    v = torch.randn(1, 1, 128, 128, generator=gen).to(torch.bfloat16).to(dev)
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 1, g, 1, 1, n_bf16=16, n_u4=32,
                          select_mode=kvq.KVQ_SELECT_THRESHOLD, tau_bf16=2.5, tau_u4=2.0)
    mask = torch.zeros(160, dtype=torch.uint8, device=dev)
    kvq.kvq_select_channels(cfg, q, lq, k, 128, mask)
    pb = kvq.kvq_page_bytes(cfg)
    arena = torch.zeros(pb, dtype=torch.uint8, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    kvq.kvq_flush_quantize(cfg, k, v, 128, 1, mask, None, arena, 0, flags)
    qd = torch.randn(1, g, 128, generator=gen).to(torch.bfloat16).to(dev)
    out = torch.zeros(1, g, 128, dtype=torch.float32, device=dev)
    ws_bytes = kvq.kvq_workspace_bytes(cfg, 1)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
    kvq.kvq_decode_attention(cfg, qd, arena, 1, mask, None, None, None, 0, None, None, 0, 0, 1 / math.sqrt(128), out,
                             ws, ws_bytes)
    torch.cuda.synchronize()
    kb = synth.bf16_bits(k[0, 0])
    tier, perm, _, n16, n4 = osel.mixkvq_threshold_select(synth.bf16_bits(q[0]), kb, 16, 32, 2.5, 2.0)
    assert (n16, n4) == (8, 24)
    rec = osel.mixkvq_record(tier, perm)
    assert np.array_equal(mask.cpu().numpy(), rec)
    page = oflush.flush_mixkvq_page(kb, synth.bf16_bits(v[0, 0]), perm, n16, n4)
    assert np.array_equal(arena.cpu().numpy()[:page.size], page)
    ref, _ = oatt.decode_arena_head(0, synth.bf16_bits(qd[0]), [page], 1 / math.sqrt(128), n16=n16, n4=n4,
                                    perm=perm)
    assert np.all(rel_err(out[0].cpu().numpy(), ref) <= TOL)
