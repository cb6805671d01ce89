"""KIVI's Value FIFO on the GPU (KIVI blog sections 4-6): Keys sealed a whole
128-token segment at a time (kvq_flush_keys), Values leaving the
full-precision window one token at a time (kvq_value_push), and decodes
whose Key boundary and Value boundary differ (kvq_decode_attention_fifo), in
the fixed flash order of section 5 (append, attend, seal a full Key segment,
move the oldest Value out). Every decode step's output is checked against
the oracle on two (batch, kv head) slices, and the pages at the end bit for
bit against the oracle's pages with their pushed Value rows.
"""
import math

import numpy as np
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import rel_err
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import flush as oflush
from oracle import layout as olayout
from oracle import select as osel

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

TOL = 2e-3
D = 128
R = 128


def bits(t):
    return synth.bf16_bits(t)


@pytest.mark.parametrize("name", ["llama8b_8k", "pnmix_16k", "qjl_32k"])
def test_fifo_decode_flow(name):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=4, n_resid=0, n_sink=0,
                    seed=base.seed + 1200)
    P, S = 200, 100                       # prefill tokens, decode steps
    L = w.n_pages * 128                   # the token stream (512 rows per head)
    g, H = w.group, w.batch * w.n_kv_heads
    print(f"\n[case] fifo {w}", flush=True)
    dev = "cuda"
    cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, w.n_pages, n_bf16=w.n_bf16, n_u4=w.n_u4,
                          n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m)
    q_pre, k, v = synth.prefill(w, dev)
    Sm = synth.qjl_matrix(w, dev) if w.key_mode == synth.QJL else None
    mb = kvq.kvq_mask_bytes(cfg)
    mask = torch.zeros(max(1, H * mb), dtype=torch.uint8, device=dev)
    if w.key_mode != synth.QJL:           # selection over the prefill's first Key segment
        kvq.kvq_select_channels(cfg, q_pre, 128, k, 128, mask, q_stride=L, k_stride=L)
    pb = kvq.kvq_page_bytes(cfg)
    arena = torch.zeros(H * w.n_pages * pb, dtype=torch.uint8, device=dev)
    flags = torch.zeros(4, dtype=torch.int32, device=dev)
    ws_bytes = kvq.kvq_workspace_bytes(cfg, w.n_pages)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
    out = torch.zeros(w.batch, w.n_q_heads, D, dtype=torch.float32, device=dev)
    kp, vp = k.data_ptr(), v.data_ptr()
    row = 128 * 2                          # bytes per token row

    # the prefill's persisted state (KIVI blog section 5, state after P tokens)
    tk = R * (P // R)                      # sealed Key tokens
    n_vq = P - min(P, R)                   # quantized Values
    for pg in range(tk // R):
        kvq.kvq_flush_keys(cfg, kp + pg * R * row, kp + pg * R * row, L, 1, mask, Sm, arena, pg, flags)
    if n_vq:
        kvq.kvq_value_push(cfg, vp, L, n_vq, 0, mask, arena, flags)

    # oracle side: the records, the sealed pages (Values added as they leave)
    kb = {(b, h): bits(k[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
    vb = {(b, h): bits(v[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
    heads = [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]
    recs, geo_off_v = {}, None
    for b, h in heads:
        if w.key_mode == synth.MIXKVQ:
            tier, perm, _ = osel.mixkvq_select(bits(q_pre[b, h * g:(h + 1) * g, :128]), kb[(b, h)][:128], w.n_bf16,
                                               w.n_u4)
            recs[(b, h)] = osel.mixkvq_record(tier, perm)
            geo_off_v = olayout.mixkvq_geometry(w.n_bf16, w.n_u4)["off_v"]
        elif w.key_mode == synth.PNMIX:
            recs[(b, h)] = osel.pnmix_select(bits(q_pre[b, h * g:(h + 1) * g, :128]), kb[(b, h)][:128],
                                             w.n_hi_pairs)[2]
            geo_off_v = olayout.pnmix_geometry(2 * w.n_hi_pairs)["off_v"]
        else:
            recs[(b, h)] = None
            geo_off_v = olayout.qjl_geometry(w.qjl_m)["off_v"]
    s_bits = bits(Sm) if Sm is not None else None

    def oracle_full_page(b, h, pg):
        kk, vv = kb[(b, h)][128 * pg:128 * pg + 128], vb[(b, h)][128 * pg:128 * pg + 128]
        if w.key_mode == synth.MIXKVQ:
            return oflush.flush_mixkvq_page(kk, vv, recs[(b, h)][:128], w.n_bf16, w.n_u4)
        if w.key_mode == synth.PNMIX:
            return oflush.flush_pnmix_page(kk, vv, osel.hi_channels_from_record(recs[(b, h)]))
        return oflush.flush_qjl_page(kk, vv, s_bits)

    full_pages = {(b, h): [oracle_full_page(b, h, pg) for pg in range(w.n_pages)] for b, h in heads}

    def oracle_pages(b, h, tk, n_vq):
        return [oatt.fifo_page(full_pages[(b, h)][pg], geo_off_v, min(R, max(0, n_vq - R * pg)))
                for pg in range(tk // R)]

    worst = 0.0
    for s in range(S):
        n = P + s                          # the new token's index; n + 1 tokens visible
        st = ocache.flash_step(R, n + 1)   # section 5 state at this step
        assert st.k_compute_full == n + 1 - tk and st.v_compute_full == n + 1 - n_vq
        qd = synth.decode_query(w, dev, step=s)
        kvq.kvq_decode_attention_fifo(cfg, qd, arena, tk // R, n_vq, mask, Sm, kp + tk * row, n + 1 - tk, L,
                                      vp + n_vq * row, n + 1 - n_vq, L, 1 / math.sqrt(D), out, ws, ws_bytes)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        for b, h in heads:
            kw = dict(n16=w.n_bf16, n4=w.n_u4, s_bits=s_bits)
            if w.key_mode == synth.MIXKVQ:
                kw["perm"] = recs[(b, h)][:128]
            elif w.key_mode == synth.PNMIX:
                kw["mask_rec"] = recs[(b, h)]
            ref, _ = oatt.decode_arena_head(w.key_mode, bits(qd[b, h * g:(h + 1) * g]), oracle_pages(b, h, tk, n_vq),
                                            1 / math.sqrt(D), resid_k=kb[(b, h)][tk:n + 1], n_vq=n_vq,
                                            vwin=vb[(b, h)][n_vq:n + 1], **kw)
            err = rel_err(o[b, h * g:(h + 1) * g], ref)
            worst = max(worst, float(err.max()))
            assert np.all(err <= TOL), (name, s, b, h, err)
        # after the step: seal a full Key segment, move the oldest Value out
        if n + 1 - tk == R:
            kvq.kvq_flush_keys(cfg, kp + tk * row, kp + tk * row, L, 1, mask, Sm, arena, tk // R, flags)
            tk += R
        if n + 1 - n_vq > R:
            kvq.kvq_value_push(cfg, vp + n_vq * row, L, 1, n_vq, mask, arena, flags)
            n_vq += 1
    torch.cuda.synchronize()
    assert int(flags[0].item()) == 0
    a = arena.cpu().numpy().reshape(H, w.n_pages, pb)
    for b, h in heads:
        for pg, ref in enumerate(oracle_pages(b, h, tk, n_vq)):
            assert np.array_equal(a[b * w.n_kv_heads + h, pg][:ref.size], ref), (name, b, h, pg)
    print(f"[fifo] {name}: {S} steps, sealed {tk} Key tokens, {n_vq} quantized Values, worst error {worst:.2e}")
