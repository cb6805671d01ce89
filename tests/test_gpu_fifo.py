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
split; and single decodes in the states the flows do not reach (no sealed
page at all, a window over every sealed page, a window of 252 tokens).
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
ROW = 128 * 2                             # bytes per bf16 token row


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


class FifoRig:
    """A Value-FIFO cache of workload w on the GPU (its records selected over
    the prefill's first Key segment) and the oracle's view of two of its
    (batch, kv head) slices. paged: a second arena reached through a random
    permutation of the pool, kept beside the contiguous one."""

    def __init__(self, w, tau=None, paged=False):
        self.w, self.tau = w, tau
        self.L = L = w.n_pages * 128      # the token stream (rows per head)
        self.g, H = w.group, w.batch * w.n_kv_heads
        dev = "cuda"
        self.q_pre, self.k, self.v = q_pre, k, v = synth.prefill(w, dev)
        self.cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, w.n_pages, n_bf16=w.n_bf16,
                                   n_u4=w.n_u4, n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m, qjl_outliers=w.qjl_outliers,
                                   qjl_m_out=w.qjl_m_out,
                                   select_mode=kvq.KVQ_SELECT_THRESHOLD if tau else kvq.KVQ_SELECT_COUNT,
                                   tau_bf16=tau[0] if tau else 0.0, tau_u4=tau[1] if tau else 0.0)
        self.cfg_generic = kvq.with_fields(self.cfg, decode_path=kvq.KVQ_DECODE_GENERIC)
        self.Sm = Sm = synth.qjl_matrix(w, dev) if w.key_mode == synth.QJL else None
        self.mb = mb = kvq.kvq_mask_bytes(self.cfg)
        self.mask = torch.zeros(max(1, H * mb), dtype=torch.uint8, device=dev)
        if w.key_mode != synth.QJL:       # selection over the prefill's first Key segment
            kvq.kvq_select_channels(self.cfg, q_pre, 128, k, 128, self.mask, q_stride=L, k_stride=L)
        elif w.qjl_outliers:              # outlier channels from the same segment's Keys
            kvq.kvq_select_channels(self.cfg, None, 0, k, 128, self.mask, k_stride=L)
        self.pb = pb = kvq.kvq_page_bytes(self.cfg)
        self.flags = torch.zeros(4, dtype=torch.int32, device=dev)
        self.ws_bytes = kvq.kvq_workspace_bytes(self.cfg, w.n_pages)
        self.ws = torch.zeros(self.ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
        self.kp, self.vp = k.data_ptr(), v.data_ptr()
        self.runs = [dict(arena=torch.zeros(H * w.n_pages * pb, dtype=torch.uint8, device=dev), table=None,
                          out=torch.zeros(w.batch, w.n_q_heads, D, dtype=torch.float32, device=dev))]
        if paged:
            gen = torch.Generator(device="cpu").manual_seed(w.seed)
            table = torch.randperm(H * w.n_pages, generator=gen).to(torch.int32).reshape(H, w.n_pages)
            self.runs.append(dict(arena=torch.zeros_like(self.runs[0]["arena"]), table=table.to(dev),
                                  out=torch.zeros_like(self.runs[0]["out"])))
        self.out_generic = torch.zeros_like(self.runs[0]["out"])
        self._oracle_side()

    def tab(self, r):
        return dict(page_table=r["table"], table_stride=self.w.n_pages if r["table"] is not None else 0)

    def seal(self, tok, page):
        for r in self.runs:
            kvq.kvq_flush_keys(self.cfg, self.kp + tok * ROW, self.kp + tok * ROW, self.L, 1, self.mask, self.Sm,
                               r["arena"], page, self.flags, **self.tab(r))

    def push(self, first, n_rows):
        for r in self.runs:
            kvq.kvq_value_push(self.cfg, self.vp + first * ROW, self.L, n_rows, first, self.mask, r["arena"],
                               self.flags, **self.tab(r))

    def _oracle_side(self):
        """The records, the full pages and the decode arguments of two slices."""
        w, g = self.w, self.g
        self.kb = {(b, h): bits(self.k[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
        self.vb = {(b, h): bits(self.v[b, h]) for b in range(w.batch) for h in range(w.n_kv_heads)}
        self.heads = [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]
        s_bits = bits(self.Sm) if self.Sm is not None else None
        self.off_v, self.dkw, full = {}, {}, {}
        for b, h in self.heads:
            kb, vb = self.kb[(b, h)], self.vb[(b, h)]
            qb = bits(self.q_pre[b, h * g:(h + 1) * g, :128])
            if w.key_mode == synth.MIXKVQ:
                if self.tau:
                    tier, perm = osel.mixkvq_threshold_select(qb, kb[:128], w.n_bf16, w.n_u4, *self.tau)[:2]
                else:
                    tier, perm, _ = osel.mixkvq_select(qb, kb[:128], w.n_bf16, w.n_u4)
                rec = osel.mixkvq_record(tier, perm)
                n16, n4 = osel.record_counts(rec) if self.tau else (w.n_bf16, w.n_u4)
                self.off_v[(b, h)] = olayout.mixkvq_geometry(n16, n4)["off_v"]
                self.dkw[(b, h)] = dict(n16=n16, n4=n4, perm=rec[:128])
                page = lambda kk, vv, rec=rec, n16=n16, n4=n4: oflush.flush_mixkvq_page(kk, vv, rec[:128], n16, n4)
            elif w.key_mode == synth.PNMIX:
                rec = osel.pnmix_select(qb, kb[:128], w.n_hi_pairs)[2]
                self.off_v[(b, h)] = olayout.pnmix_geometry(2 * w.n_hi_pairs)["off_v"]
                self.dkw[(b, h)] = dict(mask_rec=rec)
                page = lambda kk, vv, rec=rec: oflush.flush_pnmix_page(kk, vv, osel.hi_channels_from_record(rec))
            elif w.qjl_outliers:
                rec = oqjl.outlier_record(oqjl.outlier_mask(kb[:128], w.qjl_outliers))
                outl = oqjl.outlier_mask_from_record(rec)
                self.off_v[(b, h)] = olayout.qjl_geometry(w.qjl_m, w.qjl_m_out)["off_v"]
                self.dkw[(b, h)] = dict(s_bits=s_bits, qjl_m=w.qjl_m, outl=outl)
                page = lambda kk, vv, outl=outl: oflush.flush_qjl_page(kk, vv, s_bits, m=w.qjl_m, outl=outl)
            else:
                rec = None
                self.off_v[(b, h)] = olayout.qjl_geometry(w.qjl_m)["off_v"]
                self.dkw[(b, h)] = dict(s_bits=s_bits)
                page = lambda kk, vv: oflush.flush_qjl_page(kk, vv, s_bits)
            if self.mb:                   # the GPU's record is the oracle's
                i = b * w.n_kv_heads + h
                assert np.array_equal(self.mask[i * self.mb:(i + 1) * self.mb].cpu().numpy(), rec), (b, h)
            full[(b, h)] = [page(kb[128 * pg:128 * pg + 128], vb[128 * pg:128 * pg + 128]) for pg in range(w.n_pages)]
        self.full = full

    def oracle_pages(self, b, h, tk, n_vq):
        return [oatt.fifo_page(self.full[(b, h)][pg], self.off_v[(b, h)], min(R, max(0, n_vq - R * pg)))
                for pg in range(tk // R)]

    def decode_check(self, tk, n_vq, T, qd, tag):
        """Decode the T visible tokens (tk sealed Key tokens, Values below
        n_vq quantized) on the default and the generic path; every arena's
        default output equal, both within the bound of the oracle. Returns
        the worst error."""
        w, g = self.w, self.g
        for c, r, o in [(self.cfg, r, r["out"]) for r in self.runs] + [(self.cfg_generic, self.runs[0],
                                                                         self.out_generic)]:
            kvq.kvq_decode_attention_fifo(c, qd, r["arena"], tk // R, n_vq, self.mask, self.Sm,
                                          self.kp + tk * ROW, T - tk, self.L, self.vp + n_vq * ROW, T - n_vq, self.L,
                                          1 / math.sqrt(D), o, self.ws, self.ws_bytes, **self.tab(r))
        torch.cuda.synchronize()
        for r in self.runs[1:]:
            assert torch.equal(r["out"], self.runs[0]["out"]), tag
        outs = {"default": self.runs[0]["out"].cpu().numpy(), "generic": self.out_generic.cpu().numpy()}
        worst = 0.0
        for b, h in self.heads:
            kb, vb = self.kb[(b, h)], self.vb[(b, h)]
            ref, _ = oatt.decode_arena_head(w.key_mode, bits(qd[b, h * g:(h + 1) * g]),
                                            self.oracle_pages(b, h, tk, n_vq), 1 / math.sqrt(D),
                                            resid_k=kb[tk:T], n_vq=n_vq, vwin=vb[n_vq:T], **self.dkw[(b, h)])
            for path, o in outs.items():
                err = rel_err(o[b, h * g:(h + 1) * g], ref)
                worst = max(worst, float(err.max()))
                assert np.all(err <= TOL), (tag, path, b, h, err)
        return worst

    def pages_check(self, tk, n_vq, tag):
        H, pb = self.w.batch * self.w.n_kv_heads, self.pb
        for r in self.runs:
            a = r["arena"].cpu().numpy().reshape(H * self.w.n_pages, pb)
            t = r["table"].cpu().numpy() if r["table"] is not None else None
            for b, h in self.heads:
                hi = b * self.w.n_kv_heads + h
                for pg, ref in enumerate(self.oracle_pages(b, h, tk, n_vq)):
                    slot = int(t[hi, pg]) if t is not None else hi * self.w.n_pages + pg
                    assert np.array_equal(a[slot][:ref.size], ref), (tag, b, h, pg)


@pytest.mark.parametrize("name,variant", CASES)
def test_fifo_decode_flow(name, variant):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=8 if variant == "long" else 4,
                    n_resid=0, n_sink=0, seed=base.seed + 1200 + (7 if variant != "count" else 0))
    if variant == "threshold":
        w = w.scaled(n_bf16=32, n_u4=64)
    P, S = {"long": 700, "wide": 300}.get(variant, 200), 100   # prefill tokens, decode steps
    RV = 200 if variant == "wide" else R  # Value window (Key segments stay R = 128 tokens)
    print(f"\n[case] fifo {variant} {w}", flush=True)
    tau = None
    if variant == "threshold":             # quantiles of the same (device-generated) prefill
        q_pre, k, _ = synth.prefill(w, "cuda")
        tau = threshold_taus(q_pre.cpu(), k.cpu(), w, (0.93, 0.7))
    rig = FifoRig(w, tau=tau, paged=variant == "paged")

    # the prefill's persisted state (KIVI blog section 5, state after P tokens)
    tk = R * (P // R)                      # sealed Key tokens
    n_vq = P - min(P, RV)                  # quantized Values
    for pg in range(tk // R):
        rig.seal(pg * R, pg)
    if n_vq:
        rig.push(0, n_vq)

    worst = 0.0
    for s in range(S):
        n = P + s                          # the new token's index; n + 1 tokens visible
        if RV == R:                        # section 5 state at this step
            st = ocache.flash_step(R, n + 1)
            assert st.k_compute_full == n + 1 - tk and st.v_compute_full == n + 1 - n_vq
        worst = max(worst, rig.decode_check(tk, n_vq, n + 1, synth.decode_query(w, "cuda", step=s),
                                            (name, variant, s)))
        # after the step: seal a full Key segment, move the oldest Value out
        if n + 1 - tk == R:
            rig.seal(tk, tk // R)
            tk += R
        if n + 1 - n_vq > RV:
            rig.push(n_vq, 1)
            n_vq += 1
    torch.cuda.synchronize()
    assert int(rig.flags[0].item()) == 0
    rig.pages_check(tk, n_vq, (name, variant))
    print(f"[fifo] {name} {variant}: {S} steps, sealed {tk} Key tokens, {n_vq} quantized Values, "
          f"worst error {worst:.2e}")


EDGE = [
    # (sealed Key tokens, quantized Values, visible tokens)
    (0, 0, 50),       # no sealed page: every token in the Key residual and the window
    (128, 0, 228),    # the window over the whole sealed page and the Key residual (228 rows)
    (256, 256, 300),  # no window token inside the pages
    (256, 48, 300),   # a window of 252 tokens: two window pages, 208 of its tokens inside them
    (384, 384, 384),  # no residual, no window
]


@pytest.mark.parametrize("name", ["llama8b_8k", "pnmix_16k", "qjl_outlier_32k"])
def test_fifo_edge_states(name):
    """Single FIFO decodes in states the flows do not reach, on both paths
    against the oracle; the pages of the last state bit for bit."""
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=4, n_resid=0, n_sink=0,
                    seed=base.seed + 1250)
    print(f"\n[case] fifo edges {w}", flush=True)
    for tk, n_vq, T in EDGE:
        rig = FifoRig(w)
        for pg in range(tk // R):
            rig.seal(pg * R, pg)
        if n_vq:
            rig.push(0, n_vq)
        err = rig.decode_check(tk, n_vq, T, synth.decode_query(w, "cuda"), (name, tk, n_vq, T))
        assert int(rig.flags[0].item()) == 0
        rig.pages_check(tk, n_vq, (name, tk, n_vq, T))
        print(f"[fifo edge] {name} sealed {tk} quantized {n_vq} visible {T}: worst error {err:.2e}")
