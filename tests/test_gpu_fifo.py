"""KIVI's Value FIFO on the GPU (KIVI blog sections 4-6): Keys sealed a whole
128-token segment at a time (kvq_flush_keys), Values leaving the
full-precision window one token at a time (kvq_value_push), and decodes
whose Key boundary and Value boundary differ (kvq_decode_attention_fifo), in
the fixed flash order of section 5 (append, attend, seal a full Key segment,
move the oldest Value out). Every decode step's output is checked against
the oracle on two (batch, kv head) slices, and the pages at the end bit for
bit against the oracle's pages with their pushed Value rows. Each decode
runs twice: on the default path (the pipelined kernel over the pages whose
Values are all quantized and the Key residual, the generic kernel over the
window's pages) and on the generic path alone. Cases: each Key mode; a
longer stream (several all-quantized pages before the window); a 200-token
Value window (wider than a page: the window tokens inside the pages then
span two pages, up to 200 of them); pages reached
through a page table (a random permutation of the pool), run beside the
contiguous arena and equal to it bit for bit at every step; MixKVQ threshold
tiers (each head's page laid out by its own tier counts); the QJL outlier
split.
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
from oracle import qjl as oqjl
from oracle import select as osel

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

TOL = 2e-3
D = 128
R = 128


def bits(t):
    return synth.bf16_bits(t)


CASES = [
    # (workload, variant)
    ("llama8b_8k", "count"),
    ("llama8b_8k", "long"),
    ("pnmix_16k", "count"),
    ("qjl_32k", "count"),
    ("llama8b_8k", "paged"),
    ("llama8b_8k", "threshold"),
    ("qjl_outlier_32k", "count"),
    ("llama8b_8k", "wide"),
    ("pnmix_16k", "wide"),
    ("qjl_outlier_32k", "wide"),
]


def threshold_taus(q_pre, k, w, qs):
    """Thresholds at quantiles of A_d over every (batch, kv head)'s first Key
    segment (the oracle's salience, on the host)."""
    g = w.group
    vals = []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            vals += [float(a) for a in osel.mixkvq_salience(bits(q_pre[b, h * g:(h + 1) * g, :128]),
                                                            bits(k[b, h, :128]))]
    return tuple(float(np.quantile(vals, x)) for x in qs)


@pytest.mark.parametrize("name,variant", CASES)
def test_fifo_decode_flow(name, variant):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=8 if variant == "long" else 4,
                    n_resid=0, n_sink=0, seed=base.seed + 1200 + (7 if variant != "count" else 0))
    if variant == "threshold":
        w = w.scaled(n_bf16=32, n_u4=64)
    P, S = {"long": 700, "wide": 300}.get(variant, 200), 100   # prefill tokens, decode steps
    RV = 200 if variant == "wide" else R  # Value window (Key segments stay R = 128 tokens)
    L = w.n_pages * 128                   # the token stream (rows per head)
    g, H = w.group, w.batch * w.n_kv_heads
    print(f"\n[case] fifo {variant} {w}", flush=True)
    dev = "cuda"
    q_pre, k, v = synth.prefill(w, dev)
    tau = threshold_taus(q_pre.cpu(), k.cpu(), w, (0.93, 0.7)) if variant == "threshold" else None
    cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, w.n_pages, n_bf16=w.n_bf16, n_u4=w.n_u4,
                          n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m, qjl_outliers=w.qjl_outliers,
                          qjl_m_out=w.qjl_m_out,
                          select_mode=kvq.KVQ_SELECT_THRESHOLD if tau else kvq.KVQ_SELECT_COUNT,
                          tau_bf16=tau[0] if tau else 0.0, tau_u4=tau[1] if tau else 0.0)
    Sm = synth.qjl_matrix(w, dev) if w.key_mode == synth.QJL else None
    mb = kvq.kvq_mask_bytes(cfg)
    mask = torch.zeros(max(1, H * mb), dtype=torch.uint8, device=dev)
    if w.key_mode != synth.QJL:           # selection over the prefill's first Key segment
        kvq.kvq_select_channels(cfg, q_pre, 128, k, 128, mask, q_stride=L, k_stride=L)
    elif w.qjl_outliers:                  # outlier channels from the same segment's Keys
        kvq.kvq_select_channels(cfg, None, 0, k, 128, mask, k_stride=L)
    pb = kvq.kvq_page_bytes(cfg)
    flags = torch.zeros(4, dtype=torch.int32, device=dev)
    ws_bytes = kvq.kvq_workspace_bytes(cfg, w.n_pages)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
    kp, vp = k.data_ptr(), v.data_ptr()
    row = 128 * 2                          # bytes per token row
    # the arenas the flow runs on: contiguous, and with "paged" also one through a table
    runs = [dict(arena=torch.zeros(H * w.n_pages * pb, dtype=torch.uint8, device=dev), table=None,
                 out=torch.zeros(w.batch, w.n_q_heads, D, dtype=torch.float32, device=dev))]
    if variant == "paged":
        gen = torch.Generator(device="cpu").manual_seed(w.seed)
        table = torch.randperm(H * w.n_pages, generator=gen).to(torch.int32).reshape(H, w.n_pages)
        runs.append(dict(arena=torch.zeros_like(runs[0]["arena"]), table=table.to(dev),
                         out=torch.zeros_like(runs[0]["out"])))

    cfg_generic = kvq.with_fields(cfg, decode_path=kvq.KVQ_DECODE_GENERIC)
    out_generic = torch.zeros_like(runs[0]["out"])

    def tab(r):
        return dict(page_table=r["table"], table_stride=w.n_pages if r["table"] is not None else 0)

    def seal(tok, page):
        for r in runs:
            kvq.kvq_flush_keys(cfg, kp + tok * row, kp + tok * row, L, 1, mask, Sm, r["arena"], page, flags, **tab(r))

    def push(first, n_rows):
        for r in runs:
            kvq.kvq_value_push(cfg, vp + first * row, L, n_rows, first, mask, r["arena"], flags, **tab(r))

    # the prefill's persisted state (KIVI blog section 5, state after P tokens)
    tk = R * (P // R)                      # sealed Key tokens
    n_vq = P - min(P, RV)                  # quantized Values
    for pg in range(tk // R):
        seal(pg * R, pg)
    if n_vq:
        push(0, n_vq)

    # oracle side: the records, the sealed pages (Values added as they leave)
    kb = {(b, h): bits(k[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
    vb = {(b, h): bits(v[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
    heads = [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]
    s_bits = bits(Sm) if Sm is not None else None
    recs, off_v, dkw = {}, {}, {}
    for b, h in heads:
        qb = bits(q_pre[b, h * g:(h + 1) * g, :128])
        if w.key_mode == synth.MIXKVQ:
            if tau:
                tier, perm = osel.mixkvq_threshold_select(qb, kb[(b, h)][:128], w.n_bf16, w.n_u4, *tau)[:2]
            else:
                tier, perm, _ = osel.mixkvq_select(qb, kb[(b, h)][:128], w.n_bf16, w.n_u4)
            rec = osel.mixkvq_record(tier, perm)
            n16, n4 = osel.record_counts(rec) if tau else (w.n_bf16, w.n_u4)
            off_v[(b, h)] = olayout.mixkvq_geometry(n16, n4)["off_v"]
            dkw[(b, h)] = dict(n16=n16, n4=n4, perm=rec[:128])
        elif w.key_mode == synth.PNMIX:
            rec = osel.pnmix_select(qb, kb[(b, h)][:128], w.n_hi_pairs)[2]
            off_v[(b, h)] = olayout.pnmix_geometry(2 * w.n_hi_pairs)["off_v"]
            dkw[(b, h)] = dict(mask_rec=rec)
        elif w.qjl_outliers:
            rec = oqjl.outlier_record(oqjl.outlier_mask(kb[(b, h)][:128], w.qjl_outliers))
            off_v[(b, h)] = olayout.qjl_geometry(w.qjl_m, w.qjl_m_out)["off_v"]
            dkw[(b, h)] = dict(s_bits=s_bits, qjl_m=w.qjl_m, outl=oqjl.outlier_mask_from_record(rec))
        else:
            rec = None
            off_v[(b, h)] = olayout.qjl_geometry(w.qjl_m)["off_v"]
            dkw[(b, h)] = dict(s_bits=s_bits)
        recs[(b, h)] = rec
        if mb:                             # the GPU's record is the oracle's
            gpu_rec = mask[(b * w.n_kv_heads + h) * mb:(b * w.n_kv_heads + h + 1) * mb].cpu().numpy()
            assert np.array_equal(gpu_rec, rec), (name, variant, b, h)

    def oracle_full_page(b, h, pg):
        kk, vv = kb[(b, h)][128 * pg:128 * pg + 128], vb[(b, h)][128 * pg:128 * pg + 128]
        rec = recs[(b, h)]
        if w.key_mode == synth.MIXKVQ:
            return oflush.flush_mixkvq_page(kk, vv, rec[:128], dkw[(b, h)]["n16"], dkw[(b, h)]["n4"])
        if w.key_mode == synth.PNMIX:
            return oflush.flush_pnmix_page(kk, vv, osel.hi_channels_from_record(rec))
        if w.qjl_outliers:
            return oflush.flush_qjl_page(kk, vv, s_bits, m=w.qjl_m, outl=dkw[(b, h)]["outl"])
        return oflush.flush_qjl_page(kk, vv, s_bits)

    full_pages = {(b, h): [oracle_full_page(b, h, pg) for pg in range(w.n_pages)] for b, h in heads}

    def oracle_pages(b, h, tk, n_vq):
        return [oatt.fifo_page(full_pages[(b, h)][pg], off_v[(b, h)], min(R, max(0, n_vq - R * pg)))
                for pg in range(tk // R)]

    worst = 0.0
    for s in range(S):
        n = P + s                          # the new token's index; n + 1 tokens visible
        if RV == R:                        # section 5 state at this step
            st = ocache.flash_step(R, n + 1)
            assert st.k_compute_full == n + 1 - tk and st.v_compute_full == n + 1 - n_vq
        qd = synth.decode_query(w, dev, step=s)
        for c, r, o in [(cfg, r, r["out"]) for r in runs] + [(cfg_generic, runs[0], out_generic)]:
            kvq.kvq_decode_attention_fifo(c, qd, r["arena"], tk // R, n_vq, mask, Sm, kp + tk * row, n + 1 - tk,
                                          L, vp + n_vq * row, n + 1 - n_vq, L, 1 / math.sqrt(D), o, ws,
                                          ws_bytes, **tab(r))
        torch.cuda.synchronize()
        for r in runs[1:]:
            assert torch.equal(r["out"], runs[0]["out"]), (name, variant, s)
        outs = {"default": runs[0]["out"].cpu().numpy(), "generic": out_generic.cpu().numpy()}
        for b, h in heads:
            ref, _ = oatt.decode_arena_head(w.key_mode, bits(qd[b, h * g:(h + 1) * g]), oracle_pages(b, h, tk, n_vq),
                                            1 / math.sqrt(D), resid_k=kb[(b, h)][tk:n + 1], n_vq=n_vq,
                                            vwin=vb[(b, h)][n_vq:n + 1], **dkw[(b, h)])
            for tag, o in outs.items():
                err = rel_err(o[b, h * g:(h + 1) * g], ref)
                worst = max(worst, float(err.max()))
                assert np.all(err <= TOL), (name, variant, tag, s, b, h, err)
        # after the step: seal a full Key segment, move the oldest Value out
        if n + 1 - tk == R:
            seal(tk, tk // R)
            tk += R
        if n + 1 - n_vq > RV:
            push(n_vq, 1)
            n_vq += 1
    torch.cuda.synchronize()
    assert int(flags[0].item()) == 0
    for r in runs:
        a = r["arena"].cpu().numpy().reshape(H * w.n_pages, pb)
        t = r["table"].cpu().numpy() if r["table"] is not None else None
        for b, h in heads:
            hi = b * w.n_kv_heads + h
            for pg, ref in enumerate(oracle_pages(b, h, tk, n_vq)):
                slot = int(t[hi, pg]) if t is not None else hi * w.n_pages + pg
                assert np.array_equal(a[slot][:ref.size], ref), (name, variant, b, h, pg)
    print(f"[fifo] {name} {variant}: {S} steps, sealed {tk} Key tokens, {n_vq} quantized Values, "
          f"worst error {worst:.2e}")
