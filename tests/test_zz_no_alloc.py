"""kvq_decode_attention_noalloc (the decode for callers that cannot allocate:
its scratch is the library's per-GPU array) against kvq_decode_attention with
a caller-owned workspace: bit-identical outputs on two calls in a row, the
second with a smaller input, for a MixKVQ and a QJL cache (whose S q also
lives in the scratch); a call needing more scratch than the array holds is
rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import Pipeline

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]


def both(p, n_pages, n_resid):
    """(workspace decode, allocation-free decode) outputs of pipeline p."""
    w = p.w
    p.decode(n_pages=n_pages, n_resid=n_resid)
    torch.cuda.synchronize()
    ref = p.out.clone()
    out = torch.full_like(p.out, float("nan"))
    kvq.kvq_decode_attention_noalloc(p.cfg, p.q_dec, p.arena, n_pages, p.mask, p.S, p.sink_k, p.sink_v, w.n_sink,
                                     p.resid_k, p.resid_v, n_resid, 128, p.scale, out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("name", ["llama8b_8k", "qjl_32k"])
def test_noalloc_matches_workspace_decode(name):
    base = synth.WORKLOADS[name]
    big = base.scaled(batch=4, n_pages=12, seed=base.seed + 500)
    small = base.scaled(batch=1, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=3, seed=base.seed + 501)
    for w, n_pages, n_resid in ((big, big.n_pages, big.n_resid), (small, 2, min(small.n_resid, 17))):
        print(f"\n[case] noalloc {w} n_pages={n_pages} n_resid={n_resid}", flush=True)
        assert kvq.kvq_workspace_bytes(Pipeline(w, need_q_pre=False).cfg, n_pages) <= kvq.KVQ_NOALLOC_SCRATCH_BYTES
        p = Pipeline(w)
        p.select()
        p.flush_prefill()
        ref, out = both(p, n_pages, n_resid)
        assert torch.equal(ref, out), name
        assert np.all(np.isfinite(out.cpu().numpy()))


def test_noalloc_rejects_oversized_call():
    w = synth.WORKLOADS["llama8b_8k"].scaled(batch=64, n_q_heads=64, n_kv_heads=8, n_pages=1, n_resid=0)
    cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, 2, n_bf16=w.n_bf16, n_u4=w.n_u4)
    assert kvq.kvq_workspace_bytes(cfg, 1) > kvq.KVQ_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(w.batch, w.n_q_heads, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(w.batch, w.n_q_heads, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_decode_attention_noalloc(cfg, q, None, 0, None, None, None, None, 0, None, None, 0, 0, 0.088, out)
    assert e.value.status == kvq.KVQ_WORKSPACE_TOO_SMALL
