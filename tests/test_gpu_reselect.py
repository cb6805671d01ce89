"""Per-flush reselection (MixKVQ: a running accumulator of query magnitudes,
tiers refreshed for every flushed page) against the oracle: the accumulator
equals the oracle's exact query sums word for word; every reselected page's
record and bytes are the oracle's (selection from the accumulated sums and
the page's own Keys, then the flush with that order) bit for bit; the decode
with per-page records is within the decode bound of the oracle's decode with
per-page channel orders; after one decode query is accumulated, the
residual's page is reselected with the updated sums.
"""
import math

import numpy as np
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import rel_err
from oracle import attention as oatt
from oracle import flush as oflush
from oracle import select as osel

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

TOL = 2e-3
D = 128


def bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().astype(np.uint16)


def acc_ints(acc, head):
    a = acc.view(-1, D, 2)[head].cpu().numpy().astype(np.uint64)
    return [int(a[d, 0]) + (int(a[d, 1]) << 64) for d in range(D)]


@pytest.mark.parametrize("name", ["tiny_mixkvq", "llama8b_8k", "llama8b_8k_full"])
def test_reselect_flow(name):
    """llama8b_8k_full is the benchmark's reselection cache (four pages per
    decode split, so the per-page tables are rebuilt inside a split)."""
    base = synth.WORKLOADS[name.replace("_full", "")]
    if name == "tiny_mixkvq" or name.endswith("_full"):
        w = base
    else:
        w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=4, seed=base.seed + 1000)
    print(f"\n[case] reselect {w}", flush=True)
    g, H, L = w.group, w.batch * w.n_kv_heads, w.prefill_tokens
    max_pages = w.n_pages + 1
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, w.batch, w.n_q_heads, w.n_kv_heads, max_pages, n_bf16=w.n_bf16,
                          n_u4=w.n_u4, page_records=1)
    pb = kvq.kvq_page_bytes(cfg)
    q, k, v = synth.prefill(w, "cuda")
    qd = synth.decode_query(w, "cuda")
    acc = torch.zeros(H * D * 2, dtype=torch.int64, device="cuda")
    kvq.kvq_accumulate_query(cfg, q, L, L, acc)
    records = torch.zeros(H * max_pages * 160, dtype=torch.uint8, device="cuda")
    arena = torch.zeros(H * max_pages * pb, dtype=torch.uint8, device="cuda")
    flags = torch.zeros(4, dtype=torch.int32, device="cuda")
    kvq.kvq_flush_reselect(cfg, k, v, L, w.n_pages, acc, records, arena, 0, flags)
    resid_k = torch.zeros(w.batch, w.n_kv_heads, 128, D, dtype=torch.bfloat16, device="cuda")
    resid_v = torch.zeros_like(resid_k)
    t0 = w.n_pages * 128
    resid_k[:, :, :w.n_resid] = k[:, :, t0:t0 + w.n_resid]
    resid_v[:, :, :w.n_resid] = v[:, :, t0:t0 + w.n_resid]
    out = torch.zeros(w.batch, w.n_q_heads, D, dtype=torch.float32, device="cuda")
    ws_bytes = kvq.kvq_workspace_bytes(cfg, w.n_pages)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    kvq.kvq_decode_attention(cfg, qd, arena, w.n_pages, records, None, None, None, 0, resid_k, resid_v, w.n_resid,
                             128, scale, out, ws, ws_bytes)
    torch.cuda.synchronize()
    assert int(flags[0].item()) == 0
    # the pipelined kernel (when it covers the shape) against the generic one
    out_g = torch.zeros_like(out)
    kvq.kvq_decode_attention(kvq.with_fields(cfg, decode_path=kvq.KVQ_DECODE_GENERIC), qd, arena, w.n_pages, records,
                             None, None, None, 0, resid_k, resid_v, w.n_resid, 128, scale, out_g, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.all(rel_err(out.cpu().numpy().reshape(-1, D), out_g.cpu().numpy().reshape(-1, D)) <= 2 * TOL)
    rec_all = records.cpu().numpy().reshape(H, max_pages, 160)
    arena_np = arena.cpu().numpy().reshape(H, max_pages, pb)
    o = out.cpu().numpy()
    heads = [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]
    sq_of = {}
    for b, h in heads:
        head = b * w.n_kv_heads + h
        sq = osel.query_sums(bits(q[b, h * g:(h + 1) * g]))
        assert acc_ints(acc, head) == sq, (b, h)
        sq_of[(b, h)] = sq
        kb, vb = bits(k[b, h]), bits(v[b, h])
        perms, pages = [], []
        for pg in range(w.n_pages):
            tier, perm, _ = osel.mixkvq_select_sums(sq, kb[128 * pg:128 * pg + 128], w.n_bf16, w.n_u4)
            assert np.array_equal(rec_all[head, pg], osel.mixkvq_record(tier, perm)), (b, h, pg)
            ref = oflush.flush_mixkvq_page(kb[128 * pg:128 * pg + 128], vb[128 * pg:128 * pg + 128], perm, w.n_bf16,
                                           w.n_u4)
            assert np.array_equal(arena_np[head, pg], ref), (b, h, pg)
            perms.append(perm)
            pages.append(ref)
        ref_o, _ = oatt.decode_arena_head(0, bits(qd[b, h * g:(h + 1) * g]), pages, scale, n16=w.n_bf16, n4=w.n_u4,
                                          page_perms=perms, resid_k=bits(resid_k[b, h, :w.n_resid]) if w.n_resid else None,
                                          resid_v=bits(resid_v[b, h, :w.n_resid]) if w.n_resid else None)
        assert np.all(rel_err(o[b, h * g:(h + 1) * g], ref_o) <= TOL), (b, h)
    # one decode step later: its query joins the sums, the residual's page is reselected with them
    kvq.kvq_accumulate_query(cfg, qd, 1, 1, acc)
    kvq.kvq_flush_reselect(cfg, resid_k, resid_v, 128, 1, acc, records, arena, w.n_pages, flags)
    torch.cuda.synchronize()
    rec_all = records.cpu().numpy().reshape(H, max_pages, 160)
    arena_np = arena.cpu().numpy().reshape(H, max_pages, pb)
    for b, h in heads:
        head = b * w.n_kv_heads + h
        sq2 = [a + c for a, c in zip(sq_of[(b, h)], osel.query_sums(bits(qd[b, h * g:(h + 1) * g])[:, None, :]))]
        assert acc_ints(acc, head) == sq2
        rkb, rvb = bits(resid_k[b, h]), bits(resid_v[b, h])
        tier, perm, _ = osel.mixkvq_select_sums(sq2, rkb, w.n_bf16, w.n_u4)
        assert np.array_equal(rec_all[head, w.n_pages], osel.mixkvq_record(tier, perm)), (b, h)
        assert np.array_equal(arena_np[head, w.n_pages], oflush.flush_mixkvq_page(rkb, rvb, perm, w.n_bf16, w.n_u4))


@pytest.mark.parametrize("full", [False, True])
def test_reselect_through_page_table(full):
    """The same reselection flow with the pages scattered over the pool by a
    page table: records (indexed by logical page), page bytes and the decode
    output equal the contiguous run's, bit for bit (full: the llama8b_8k
    shape, four pages per decode split)."""
    base = synth.WORKLOADS["llama8b_8k"]
    w = base if full else base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=5,
                                      seed=base.seed + 1100)
    print(f"\n[case] reselect paged {w}", flush=True)
    H, L = w.batch * w.n_kv_heads, w.prefill_tokens
    max_pages = w.n_pages + 1
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, w.batch, w.n_q_heads, w.n_kv_heads, max_pages, n_bf16=w.n_bf16,
                          n_u4=w.n_u4, page_records=1)
    pb = kvq.kvq_page_bytes(cfg)
    q, k, v = synth.prefill(w, "cuda")
    qd = synth.decode_query(w, "cuda")
    acc = torch.zeros(H * D * 2, dtype=torch.int64, device="cuda")
    kvq.kvq_accumulate_query(cfg, q, L, L, acc)
    pool = H * max_pages
    gen = torch.Generator(device="cpu").manual_seed(31)
    table = torch.randperm(pool, generator=gen).to(torch.int32).reshape(H, max_pages).cuda()
    runs = []
    for tab in (None, table):
        records = torch.zeros(H * max_pages * 160, dtype=torch.uint8, device="cuda")
        arena = torch.zeros(pool * pb, dtype=torch.uint8, device="cuda")
        flags = torch.zeros(4, dtype=torch.int32, device="cuda")
        kw = {} if tab is None else {"page_table": tab, "table_stride": max_pages}
        kvq.kvq_flush_reselect(cfg, k, v, L, w.n_pages, acc, records, arena, 0, flags, **kw)
        out = torch.zeros(w.batch, w.n_q_heads, D, dtype=torch.float32, device="cuda")
        ws_bytes = kvq.kvq_workspace_bytes(cfg, w.n_pages)
        ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device="cuda")
        kvq.kvq_decode_attention(cfg, qd, arena, w.n_pages, records, None, None, None, 0, None, None, 0, 0,
                                 1.0 / math.sqrt(D), out, ws, ws_bytes, **kw)
        torch.cuda.synchronize()
        runs.append((records, arena, out))
    (rec_c, arena_c, out_c), (rec_t, arena_t, out_t) = runs
    assert torch.equal(rec_c, rec_t)
    assert torch.equal(out_c, out_t)
    tab = table.cpu().numpy()
    for h in range(H):
        for pg in range(w.n_pages):
            i = int(tab[h, pg])
            assert torch.equal(arena_t[i * pb:(i + 1) * pb], arena_c[(h * max_pages + pg) * pb:(h * max_pages + pg + 1) * pb])
