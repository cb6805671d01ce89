"""The decode call and the flush captured in a HIP graph (torch.cuda.graph)
give the same bits as the eager calls on every replay.

Each replay is separated from the next by eager library calls and device
synchronisations, and every replay is compared with the eager result: a
graph node that misbehaves only on later replays shows up here.
"""
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import Pipeline

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]


@pytest.mark.parametrize("name", ["llama8b_8k", "pnmix_16k", "qjl_32k", "qjl_outlier_32k"])
def test_graph_replays_match_eager(name):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=5, n_resid=base.n_resid and 128,
                    seed=base.seed + 300)
    print(f"\n[case] graph {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()

    def step():
        p.decode()
        kvq.kvq_flush_quantize(p.cfg, p.resid_k, p.resid_v, 128, 1, p.mask, p.S, p.arena, w.n_pages, p.flags)

    step()
    torch.cuda.synchronize()
    out_ref = p.out.clone()
    page_ref = p.arena.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        p.out.zero_()
        p.arena[:] = page_ref
        p.arena.view(w.batch * w.n_kv_heads, p.max_pages, p.page_bytes)[:, w.n_pages] = 0   # the flushed pages
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(p.out, out_ref), rep
        assert torch.equal(p.arena, page_ref), rep
        # eager work between replays
        p.decode(n_pages=2, n_resid=0)
        torch.cuda.synchronize()
