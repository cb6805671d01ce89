"""Pages reached through a page table (a block table over the arena as one
page pool) against the contiguous layout, in every Key mode: the prefill
flush written through a random permutation of the pool puts every page's
bytes, bit for bit, where its table entry says; the decode through the table
(pipelined and generic kernels) gives the contiguous decode's output bit for
bit, and the oracle's within the decode bound; the fused decode + flush call
writes the residual's page through the table; a flush entry outside the pool
writes nothing and raises KVQ_FLAG_TABLE; a decode entry outside the pool is
clamped into it.
"""

import numpy as np
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import Pipeline, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

TOL = 2e-3


def paged_copy(p, seed):
    """A second arena filled by the prefill flush through a random table over
    the whole pool; returns (arena2, table [heads, max_pages] int32 on the GPU)."""
    w = p.w
    heads = w.batch * w.n_kv_heads
    pool = heads * p.max_pages
    gen = torch.Generator(device="cpu").manual_seed(seed)
    table = torch.randperm(pool, generator=gen).to(torch.int32).reshape(heads, p.max_pages).cuda()
    arena2 = torch.zeros_like(p.arena)
    flags = torch.zeros_like(p.flags)
    kvq.kvq_flush_quantize(p.cfg, p.k_offset_ptr(p.k_pre, w.n_sink), p.k_offset_ptr(p.v_pre, w.n_sink), p.L,
                           w.n_pages, p.mask, p.S, arena2, 0, flags, page_table=table, table_stride=p.max_pages)
    torch.cuda.synchronize()
    assert int(flags[0].item()) == int(p.flags[0].item())
    return arena2, table


def pool_page(arena, p, idx):
    return arena[idx * p.page_bytes:(idx + 1) * p.page_bytes]


def decode_into(p, arena, table, n_pages, n_resid, out, generic=False):
    w = p.w
    cfg = kvq.with_fields(p.cfg, decode_path=kvq.KVQ_DECODE_GENERIC) if generic else p.cfg
    kvq.kvq_decode_attention(cfg, p.q_dec, arena, n_pages, p.mask, p.S, p.sink_k, p.sink_v, w.n_sink, p.resid_k,
                             p.resid_v, n_resid, 128, p.scale, out, p.ws, p.ws_bytes, page_table=table,
                             table_stride=p.max_pages if table is not None else 0)


@pytest.mark.parametrize("name", ["tiny_mixkvq", "llama8b_8k", "qwen32b_32k", "pnmix_16k", "qjl_32k", "qjl_outlier_32k"])
def test_paged_matches_contiguous(name):
    base = synth.WORKLOADS[name]
    w = base if name == "tiny_mixkvq" else base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=6,
                                                       seed=base.seed + 800)
    print(f"\n[case] paged {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    arena2, table = paged_copy(p, 11 + w.seed)
    heads = w.batch * w.n_kv_heads
    tab = table.cpu().numpy()
    for h in range(heads):
        for pg in range(w.n_pages):
            assert torch.equal(pool_page(arena2, p, int(tab[h, pg])), pool_page(p.arena, p, h * p.max_pages + pg)), (h, pg)
    # decode: contiguous vs through the table, bit for bit
    out_c = torch.empty_like(p.out)
    out_t = torch.empty_like(p.out)
    decode_into(p, p.arena, None, w.n_pages, w.n_resid, out_c)
    decode_into(p, arena2, table, w.n_pages, w.n_resid, out_t)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_t)
    # the generic kernel through the table, against the oracle
    out_g = torch.empty_like(p.out)
    decode_into(p, arena2, table, w.n_pages, w.n_resid, out_g, generic=True)
    torch.cuda.synchronize()
    o = out_g.cpu().numpy()
    b, hk = w.batch - 1, w.n_kv_heads - 1
    rec = p.record(b, hk)
    pages = [p.oracle_page(b, hk, pg, rec) for pg in range(w.n_pages)]
    ref, _ = p.oracle_decode(b, hk, pages, rec)
    assert np.all(rel_err(o[b, hk * p.g:(hk + 1) * p.g], ref) <= TOL)
    assert np.all(rel_err(o.reshape(-1, 128), out_c.cpu().numpy().reshape(-1, 128)) <= 2 * TOL)


@pytest.mark.parametrize("name", ["llama8b_8k", "pnmix_16k"])
def test_paged_fused_step_and_bad_entry(name):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=5, seed=base.seed + 900)
    print(f"\n[case] paged fused {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    arena2, table = paged_copy(p, 23 + w.seed)
    # contiguous fused step, then the same step through the table
    flags0 = p.flags.clone()
    p.decode_flush()
    torch.cuda.synchronize()
    out_c = p.out.clone()
    p.flags.copy_(flags0)
    kvq.kvq_decode_attention_flush(p.cfg, p.q_dec, arena2, w.n_pages, p.mask, p.S, p.sink_k, p.sink_v, w.n_sink,
                                   p.resid_k, p.resid_v, w.n_resid, 128, p.scale, p.out, p.ws, p.ws_bytes,
                                   p.resid_k, p.resid_v, 128, 1, w.n_pages, p.flags, page_table=table,
                                   table_stride=p.max_pages)
    torch.cuda.synchronize()
    assert torch.equal(p.out, out_c)
    tab = table.cpu().numpy()
    for h in range(w.batch * w.n_kv_heads):
        assert torch.equal(pool_page(arena2, p, int(tab[h, w.n_pages])),
                           pool_page(p.arena, p, h * p.max_pages + w.n_pages)), h
    # a flush entry outside the pool: nothing written, KVQ_FLAG_TABLE raised
    bad = table.clone()
    bad[1, w.n_pages] = w.batch * w.n_kv_heads * p.max_pages
    before = arena2.clone()
    flags = torch.zeros_like(p.flags)
    kvq.kvq_flush_quantize(p.cfg, p.resid_k, p.resid_v, 128, 1, p.mask, p.S, arena2, w.n_pages, flags,
                           page_table=bad, table_stride=p.max_pages)
    torch.cuda.synchronize()
    assert int(flags[0].item()) & kvq.KVQ_FLAG_TABLE
    for h in range(w.batch * w.n_kv_heads):   # the other heads' pages are rewritten with the same bytes
        if h != 1:
            assert torch.equal(pool_page(arena2, p, int(tab[h, w.n_pages])), pool_page(before, p, int(tab[h, w.n_pages])))
    assert torch.equal(arena2, before)
    # decode entries outside the pool are clamped into it (0 and the last
    # pool page): the same bits as the explicitly clamped table, both kernels
    pool = w.batch * w.n_kv_heads * p.max_pages
    wild, clamped = table.clone(), table.clone()
    wild[0, 0], clamped[0, 0] = -3, 0
    wild[1, 2], clamped[1, 2] = pool + 5, pool - 1
    for cfg in (p.cfg, kvq.with_fields(p.cfg, decode_path=kvq.KVQ_DECODE_GENERIC)):
        outs = []
        for tab_ in (wild, clamped):
            o = torch.zeros_like(p.out)
            kvq.kvq_decode_attention(cfg, p.q_dec, arena2, w.n_pages, p.mask, p.S, p.sink_k, p.sink_v, w.n_sink,
                                     p.resid_k, p.resid_v, w.n_resid, 128, p.scale, o, p.ws, p.ws_bytes,
                                     page_table=tab_, table_stride=p.max_pages)
            outs.append(o)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        assert bool(torch.isfinite(outs[0]).all())
