"""GPU test harness: drives libkvq through its Python binding on a workload
and computes the oracle's answer for chosen (batch, kv head) slices.

Test infrastructure only (it imports the oracle)."""
from __future__ import annotations

import math

import numpy as np
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from oracle import attention as oatt
from oracle import flush as oflush
from oracle import qjl as oqjl
from oracle import select as osel

D = 128


class Pipeline:
    """select -> prefill flush -> decode for one workload on the GPU."""

    def __init__(self, w: synth.Workload, device="cuda", max_pages=None, need_q_pre=True, pair_layout="half",
                 tau=None):
        """tau: (tau_bf16, tau_u4) selects the MixKVQ threshold tiers, with
        the workload's n_bf16 / n_u4 as the capacities."""
        self.w = w
        self.tau = tau
        self.dev = device
        self.g = w.group
        self.L = w.prefill_tokens
        self.pair_layout = pair_layout
        self.max_pages = max_pages or max(1, w.n_pages + 1)
        self.cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, self.max_pages,
                                   n_bf16=w.n_bf16, n_u4=w.n_u4,
                                   pair_layout=kvq.KVQ_PAIR_HALF_SPLIT if pair_layout == "half" else kvq.KVQ_PAIR_ADJACENT,
                                   n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m,
                                   qjl_outliers=w.qjl_outliers, qjl_m_out=w.qjl_m_out,
                                   select_mode=kvq.KVQ_SELECT_THRESHOLD if tau else kvq.KVQ_SELECT_COUNT,
                                   tau_bf16=tau[0] if tau else 0.0, tau_u4=tau[1] if tau else 0.0)
        self.page_bytes = kvq.kvq_page_bytes(self.cfg)
        self.mask_bytes = kvq.kvq_mask_bytes(self.cfg)
        q, k, v = synth.prefill(w, device)
        self.q_pre = q if need_q_pre else None
        self.k_pre, self.v_pre = k, v
        self.q_dec = synth.decode_query(w, device)
        self.S = synth.qjl_matrix(w, device) if w.key_mode == synth.QJL else None
        H = w.batch * w.n_kv_heads
        self.mask = torch.zeros(max(1, H * self.mask_bytes), dtype=torch.uint8, device=device)
        self.arena = torch.zeros(H * self.max_pages * self.page_bytes, dtype=torch.uint8, device=device)
        self.flags = torch.zeros(4, dtype=torch.int32, device=device)
        ns, nq = w.n_sink, w.n_pages * 128
        self.sink_k = k[:, :, :ns].contiguous() if ns else None
        self.sink_v = v[:, :, :ns].contiguous() if ns else None
        self.resid_k = torch.zeros(w.batch, w.n_kv_heads, 128, D, dtype=torch.bfloat16, device=device)
        self.resid_v = torch.zeros_like(self.resid_k)
        if w.n_resid:
            self.resid_k[:, :, :w.n_resid] = k[:, :, ns + nq: ns + nq + w.n_resid]
            self.resid_v[:, :, :w.n_resid] = v[:, :, ns + nq: ns + nq + w.n_resid]
        self.out = torch.zeros(w.batch, w.n_q_heads, D, dtype=torch.float32, device=device)
        self.ws_bytes = kvq.kvq_workspace_bytes(self.cfg, w.n_pages)
        self.ws = torch.zeros(self.ws_bytes // 4 + 64, dtype=torch.float32, device=device)
        self.scale = 1.0 / math.sqrt(D)

    # ------------------------------------------------------------ GPU calls
    def k_offset_ptr(self, tensor, tok):
        return tensor.data_ptr() + tok * D * 2

    def select(self):
        w = self.w
        if w.key_mode == synth.MIXKVQ:
            kvq.kvq_select_channels(self.cfg, self.q_pre, self.q_pre.shape[2], self.k_offset_ptr(self.k_pre, w.n_sink),
                                    w.n_pages * 128, self.mask, k_stride=self.L)
        elif w.key_mode == synth.PNMIX:
            kvq.kvq_select_channels(self.cfg, self.q_pre, self.q_pre.shape[2], self.k_pre, self.L, self.mask)
        elif w.qjl_outliers:   # QJL outlier channels from the prompt's Keys
            kvq.kvq_select_channels(self.cfg, None, 0, self.k_pre, self.L, self.mask)

    def flush_prefill(self):
        w = self.w
        kvq.kvq_flush_quantize(self.cfg, self.k_offset_ptr(self.k_pre, w.n_sink), self.k_offset_ptr(self.v_pre, w.n_sink),
                               self.L, w.n_pages, self.mask, self.S, self.arena, 0, self.flags)

    def decode(self, n_pages=None, n_resid=None, generic=False):
        """generic: the config's decode path set to the generic kernel."""
        w = self.w
        n_pages = w.n_pages if n_pages is None else n_pages
        n_resid = w.n_resid if n_resid is None else n_resid
        need = kvq.kvq_workspace_bytes(self.cfg, n_pages)
        if need > self.ws_bytes:
            self.ws_bytes = need
            self.ws = torch.zeros(need // 4 + 64, dtype=torch.float32, device=self.dev)
        cfg = kvq.with_fields(self.cfg, decode_path=kvq.KVQ_DECODE_GENERIC) if generic else self.cfg
        kvq.kvq_decode_attention(cfg, self.q_dec, self.arena, n_pages, self.mask, self.S,
                                 self.sink_k, self.sink_v, w.n_sink, self.resid_k, self.resid_v, n_resid, 128,
                                 self.scale, self.out, self.ws, self.ws_bytes)
        return self.out

    def decode_flush(self, n_pages=None, n_resid=None, first_page=None, n_flush=1):
        """kvq_decode_attention_flush: the decode of `decode`, then the
        residual buffer (all 128 rows) flushed into pages first_page .."""
        w = self.w
        n_pages = w.n_pages if n_pages is None else n_pages
        n_resid = w.n_resid if n_resid is None else n_resid
        first_page = n_pages if first_page is None else first_page
        need = kvq.kvq_workspace_bytes(self.cfg, n_pages)
        if need > self.ws_bytes:
            self.ws_bytes = need
            self.ws = torch.zeros(need // 4 + 64, dtype=torch.float32, device=self.dev)
        kvq.kvq_decode_attention_flush(self.cfg, self.q_dec, self.arena, n_pages, self.mask, self.S,
                                       self.sink_k, self.sink_v, w.n_sink, self.resid_k, self.resid_v, n_resid,
                                       128, self.scale, self.out, self.ws, self.ws_bytes, self.resid_k,
                                       self.resid_v, 128, n_flush, first_page, self.flags)
        return self.out

    # ------------------------------------------------------------ host views
    def gpu_page(self, b, h, p):
        base = ((b * self.w.n_kv_heads + h) * self.max_pages + p) * self.page_bytes
        return self.arena[base: base + self.page_bytes].cpu().numpy()

    def gpu_record(self, b, h):
        mb = self.mask_bytes
        base = (b * self.w.n_kv_heads + h) * mb
        return self.mask[base: base + mb].cpu().numpy()

    def record(self, b, h):
        """The GPU's selection record of (b, h), None where the mode has none."""
        return self.gpu_record(b, h) if self.mask_bytes else None

    def bits(self, t):
        return synth.bf16_bits(t)

    # ------------------------------------------------------------ oracle
    def oracle_record(self, b, h):
        w = self.w
        g = self.g
        if w.key_mode == synth.QJL:
            return oqjl.outlier_record(oqjl.outlier_mask(self.bits(self.k_pre[b, h]), w.qjl_outliers))
        qb = self.bits(self.q_pre[b, h * g:(h + 1) * g])
        if w.key_mode == synth.MIXKVQ:
            kb = self.bits(self.k_pre[b, h, w.n_sink: w.n_sink + w.n_pages * 128])
            if self.tau:
                tier, perm = osel.mixkvq_threshold_select(qb, kb, w.n_bf16, w.n_u4, *self.tau)[:2]
            else:
                tier, perm, _ = osel.mixkvq_select(qb, kb, w.n_bf16, w.n_u4)
            return osel.mixkvq_record(tier, perm)
        kb = self.bits(self.k_pre[b, h])
        return osel.pnmix_select(qb, kb, w.n_hi_pairs, self.pair_layout)[2]

    def oracle_page(self, b, h, p, record):
        w = self.w
        t0 = w.n_sink + 128 * p
        kb = self.bits(self.k_pre[b, h, t0:t0 + 128])
        vb = self.bits(self.v_pre[b, h, t0:t0 + 128])
        return self.oracle_flush(kb, vb, record)

    def oracle_flush(self, kb, vb, record):
        """The oracle's page of 128 tokens (bf16 bits) under a selection record."""
        w = self.w
        if w.key_mode == synth.MIXKVQ:
            return oflush.flush_mixkvq_page(kb, vb, record[:128], *self.tier_counts(record))
        if w.key_mode == synth.PNMIX:
            return oflush.flush_pnmix_page(kb, vb, osel.hi_channels_from_record(record, self.pair_layout))
        if w.qjl_outliers:
            return oflush.flush_qjl_page(kb, vb, self.bits(self.S), m=w.qjl_m,
                                         outl=oqjl.outlier_mask_from_record(record))
        return oflush.flush_qjl_page(kb, vb, self.bits(self.S))

    def oracle_decode(self, b, h, pages, record, n_resid=None):
        w = self.w
        g = self.g
        n_resid = w.n_resid if n_resid is None else n_resid
        qb = self.bits(self.q_dec[b, h * g:(h + 1) * g])
        n16, n4 = self.tier_counts(record) if w.key_mode == synth.MIXKVQ else (0, 0)
        kw = dict(n16=n16, n4=n4, perm=None if record is None else record[:128],
                  mask_rec=record, pair_layout=self.pair_layout,
                  s_bits=None if self.S is None else self.bits(self.S))
        if w.qjl_outliers:
            kw.update(qjl_m=w.qjl_m, outl=oqjl.outlier_mask_from_record(record), mask_rec=None)
        if w.n_sink:
            kw["sink_k"] = self.bits(self.k_pre[b, h, :w.n_sink])
            kw["sink_v"] = self.bits(self.v_pre[b, h, :w.n_sink])
        if n_resid:
            kw["resid_k"] = self.bits(self.resid_k[b, h, :n_resid])
            kw["resid_v"] = self.bits(self.resid_v[b, h, :n_resid])
        return oatt.decode_arena_head(w.key_mode, qb, pages, self.scale, **kw)

    def tier_counts(self, record):
        """(BF16, UINT4) counts a MixKVQ page is laid out by: the configured
        ones, or with threshold tiers the head's own (from its record)."""
        if self.tau:
            return osel.record_counts(record)
        return self.w.n_bf16, self.w.n_u4

    def same_page(self, gpu_page, oracle_page):
        """A GPU page slot holds the oracle's page (with threshold tiers the
        slot is the largest page and its tail is not written)."""
        return np.array_equal(np.asarray(gpu_page)[:oracle_page.size], oracle_page)

    def reference_probs(self, b, h, n_pages, n_resid):
        """Unquantized bf16 attention over the same visible tokens (fidelity)."""
        w = self.w
        g = self.g
        qb = self.bits(self.q_dec[b, h * g:(h + 1) * g])
        end = w.n_sink + 128 * n_pages
        kb = np.concatenate([self.bits(self.k_pre[b, h, :end]), self.bits(self.resid_k[b, h, :n_resid])])
        vb = np.concatenate([self.bits(self.v_pre[b, h, :end]), self.bits(self.resid_v[b, h, :n_resid])])
        return oatt.reference_attention(qb, kb, vb, self.scale)


def rel_err(out, ref):
    """max_d |out - ref| / max_d |ref| per query head."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.max(np.abs(out - ref), axis=-1) / np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
