"""kvq_decode_attention_flush against kvq_decode_attention followed by
kvq_flush_quantize on one stream: the decode output, every byte of the page
arena and the status bits are identical, bit for bit, in every Key mode; with
the flush target inside the decoded range (the flush writes after the decode
has read); with nothing visible; with no page to flush; and at the full
Llama-3.1-8B-shaped size the benchmark's step runs.
"""
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import Pipeline

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]


def built(w):
    print(f"\n[case] fused {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    return p


def check_fused(p, n_pages, n_resid, first_page, n_flush):
    arena0, flags0 = p.arena.clone(), p.flags.clone()
    p.out.fill_(float("nan"))
    p.decode(n_pages, n_resid)
    if n_flush:
        kvq.kvq_flush_quantize(p.cfg, p.resid_k, p.resid_v, 128, n_flush, p.mask, p.S, p.arena, first_page,
                               p.flags)
    torch.cuda.synchronize()
    out_s, arena_s, flags_s = p.out.clone(), p.arena.clone(), p.flags.clone()
    p.arena.copy_(arena0)
    p.flags.copy_(flags0)
    p.out.fill_(float("nan"))
    torch.cuda.synchronize()
    p.decode_flush(n_pages, n_resid, first_page, n_flush)
    torch.cuda.synchronize()
    assert torch.equal(p.out, out_s)
    assert torch.equal(p.arena, arena_s)
    assert torch.equal(p.flags, flags_s)


@pytest.mark.parametrize("name", ["tiny_mixkvq", "llama8b_8k", "qwen32b_32k", "pnmix_16k", "qjl_32k"])
def test_fused_matches_separate_calls(name):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=5, seed=base.seed + 700)
    p = built(w)
    check_fused(p, w.n_pages, w.n_resid, w.n_pages, 1)                    # next page
    check_fused(p, w.n_pages, w.n_resid, w.n_pages - 2, 1)                # a page the decode reads
    check_fused(p, 0, 0, 0, 1)                                            # nothing visible
    check_fused(p, w.n_pages, w.n_resid, 0, 0)                            # nothing to flush


def test_fused_full_size_step():
    w = synth.WORKLOADS["llama8b_8k"]
    p = Pipeline(w, need_q_pre=True)
    print(f"\n[case] fused full size {w}", flush=True)
    p.select()
    p.flush_prefill()
    p.q_pre = None
    torch.cuda.synchronize()
    check_fused(p, w.n_pages, w.n_resid, w.n_pages, 1)
