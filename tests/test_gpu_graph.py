"""The decode call and the flush captured in a HIP graph (torch.cuda.graph)
give the same bits as the eager calls on every replay; so does the KIVI
Value FIFO's step (FIFO decode, Value push, Key seal).

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


@pytest.mark.parametrize("name", ["llama8b_8k", "pnmix_16k", "qjl_outlier_32k"])
def test_fifo_graph_replays_match_eager(name):
    """The Value FIFO's step captured in a graph: a FIFO decode (the
    pipelined kernel, its window page's logits in spare workspace records,
    the window merge), a one-row Value push and a one-page Key seal. Every
    replay gives the eager bits."""
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=4, n_resid=0, n_sink=0,
                    seed=base.seed + 310)
    print(f"\n[case] fifo graph {w}", flush=True)
    dev = "cuda"
    L, row = w.n_pages * 128, 128 * 2
    H = w.batch * w.n_kv_heads
    cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, w.n_pages, n_bf16=w.n_bf16, n_u4=w.n_u4,
                          n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m, qjl_outliers=w.qjl_outliers, qjl_m_out=w.qjl_m_out)
    q_pre, k, v = synth.prefill(w, dev)
    Sm = synth.qjl_matrix(w, dev) if w.key_mode == synth.QJL else None
    mask = torch.zeros(max(1, H * kvq.kvq_mask_bytes(cfg)), dtype=torch.uint8, device=dev)
    if w.key_mode != synth.QJL:
        kvq.kvq_select_channels(cfg, q_pre, 128, k, 128, mask, q_stride=L, k_stride=L)
    else:
        kvq.kvq_select_channels(cfg, None, 0, k, 128, mask, k_stride=L)
    arena = torch.zeros(H * w.n_pages * kvq.kvq_page_bytes(cfg), dtype=torch.uint8, device=dev)
    flags = torch.zeros(4, dtype=torch.int32, device=dev)
    kp, vp = k.data_ptr(), v.data_ptr()
    tk, n_vq, n_kres = 256, 200, 40           # two sealed pages, 56 window tokens inside them, 40 Key-residual rows
    kvq.kvq_flush_keys(cfg, kp, kp, L, 2, mask, Sm, arena, 0, flags)
    kvq.kvq_value_push(cfg, vp, L, n_vq, 0, mask, arena, flags)
    qd = synth.decode_query(w, dev)
    out = torch.zeros(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
    ws_bytes = kvq.kvq_workspace_bytes(cfg, w.n_pages)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)

    def step():
        kvq.kvq_decode_attention_fifo(cfg, qd, arena, tk // 128, n_vq, mask, Sm, kp + tk * row, n_kres, L,
                                      vp + n_vq * row, tk + n_kres - n_vq, L, 1 / 128 ** 0.5, out, ws, ws_bytes)
        kvq.kvq_value_push(cfg, vp + n_vq * row, L, 1, n_vq, mask, arena, flags)
        kvq.kvq_flush_keys(cfg, kp + tk * row, kp + tk * row, L, 1, mask, Sm, arena, tk // 128, flags)

    state = arena.clone()
    step()
    torch.cuda.synchronize()
    out_ref, arena_ref = out.clone(), arena.clone()
    assert int(flags[0].item()) == 0
    g = torch.cuda.CUDAGraph()
    arena.copy_(state)
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        arena.copy_(state)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), rep
        assert torch.equal(arena, arena_ref), rep
        # eager work between replays
        arena.copy_(state)
        step()
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), rep
