"""Benchmark of the libkvq hot path on one MI355X.

A step is one pass of the hot path on the Llama-3.1-8B-shaped layer (batch 8,
32 query / 8 KV heads, 64 packed pages + 128 BF16 residual tokens per KV
head, MixKVQ 1/12/115 Key tiers): one decode-attention over the packed cache,
then one flush of the full 128-token residual into a new page, made as one
kvq_decode_attention_flush call (the decode kernel, then one launch holding
the flush blocks and the decode's split merge, which are independent). The
inputs (packed pages, residual, selection records, query) are resident in
HBM before the timed region. To keep the 256 MB Infinity Cache from serving
the 51 MB cache, the steps rotate over several copies of it.

The K timed steps are captured once into a HIP graph (torch.cuda.graph; the
library launches on torch's current stream, which is the capture stream) and
replayed once between two device synchronisations, so the host's per-call
launch cost is not part of the step time; `ms_per_step` is that wall time
over K. The decode call and the flush are timed the same way on their own
(K calls per graph, HIP events on the replay stream around the replay).

Prints one JSON line. `value` is the step's algorithmic packed-KV bytes
(decode reads + flush reads and writes) divided by the step time; the
decode-only GB/s, its fraction of the 8 TB/s HBM peak and the flush rate in
tokens/s are reported beside it, as is the CPU oracle on a bounded sample.
Every decode leg also reports `read_stream_GBps`: a plain read of the same
rotated cache copies by the library's read-stream reference (kvq_read_stream,
the decode kernels' load shape with nothing computed), timed the same way,
i.e. the read rate this GPU reaches at that size, and the decode's fraction
of it.
The roofline object is the decode call (decode kernel + split combine); its `traffic`
comes from profiles/decode_llama8b_8k_traffic.txt (rocprofv3 FETCH_SIZE / WRITE_SIZE
of the decode kernel, calibrated on a plain copy) and is null when the
decode sources changed since those counters were taken.

Helper modes used to make the committed profiles:
  --copy-calibration MB   run torch's copy kernel on MB megabytes (for the
                          counter calibration run under rocprofv3 --pmc)
  --summarize-pmc FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR MB
                          turn the four counter runs into
                          profiles/decode_llama8b_8k_traffic.txt
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
DECODE_SOURCES = ["mixed_precision_kv_amd/csrc/kvq_decode_fast.hip", "mixed_precision_kv_amd/csrc/kvq_decode.hip",
                  "mixed_precision_kv_amd/csrc/kvq_decode_common.h", "mixed_precision_kv_amd/csrc/kvq_internal.h",
                  "mixed_precision_kv_amd/csrc/kvq_merge.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama8b_8k_traffic.txt")
METRIC = "quantized decode-attn packed-KV GB/s (% of HBM peak); flush tokens/s"


def logical_page_bytes(w) -> int:
    """Bytes one page must hold at its logical bit widths (no padding)."""
    v = 128 * 128 * 2 // 8 + 128 * 4 * 2 * 2
    if w.key_mode == 0:
        n2 = 128 - w.n_bf16 - w.n_u4
        k = 128 * w.n_bf16 * 2 + 128 * (4 * w.n_u4 + 2 * n2) // 8 + (w.n_u4 + n2) * 2 * 2
    elif w.key_mode == 1:
        n_hi = 2 * w.n_hi_pairs
        k = 128 * 128 // 8 + 128 * n_hi * 2 // 8 + 128 * 2 * 2
    else:
        # sign bits of both instances; one binary16 norm per instance
        k = 128 * (w.qjl_m + w.qjl_m_out) // 8 + 128 * 2 * (2 if w.qjl_m_out else 1)
    return k + v


def record_bytes(w) -> int:
    return {0: 160, 1: 8, 2: 16 if w.qjl_outliers else 0}[w.key_mode]


def decode_bytes(w) -> int:
    """Algorithmic bytes of one decode call: packed pages, BF16 sinks and
    residual, the selection record, the query and the float32 output."""
    heads = w.batch * w.n_kv_heads
    g = w.group
    rec = record_bytes(w)
    per_head = (w.n_pages * logical_page_bytes(w) + (w.n_sink + w.n_resid) * 128 * 2 * 2 + rec
                + g * 128 * 2 + g * 128 * 4)
    extra = (w.qjl_m + w.qjl_m_out) * 128 * 2 if w.key_mode == 2 else 0   # S
    return heads * per_head + extra


def flush_bytes(w) -> int:
    """One 128-token flush: read K and V (bf16), read the record, write a page."""
    heads = w.batch * w.n_kv_heads
    rec = record_bytes(w)
    return heads * (128 * 128 * 2 * 2 + rec + logical_page_bytes(w))


def decode_source_sha() -> str:
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(workload: str):
    """HBM bytes per decode-kernel launch from the committed counter runs, or
    None when they are missing, for another workload, or older than the
    decode sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("decode_source_sha256") != decode_source_sha():
        return None
    return t.get("bytes_per_launch")


def _pmc_rows(d, counter):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    return rows


def summarize_pmc(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mb, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode kernel, each
    scaled by what the counter reads for torch's copy of a known size."""
    def avg(rows, pred):
        v = [float(r["Counter_Value"]) for r in rows if pred(r["Kernel_Name"])]
        return (sum(v) / len(v), len(v)) if v else (None, 0)
    is_dec = lambda n: "decode_" in n and "kvq::" in n
    is_copy = lambda n: "copybuffer" in n.lower()   # the runtime's blit kernel behind copy_()
    fk, nf = avg(_pmc_rows(fetch_dir, "FETCH_SIZE"), is_dec)
    wk, nw = avg(_pmc_rows(write_dir, "WRITE_SIZE"), is_dec)
    cf, _ = avg(_pmc_rows(copy_fetch_dir, "FETCH_SIZE"), is_copy)
    cw, _ = avg(_pmc_rows(copy_write_dir, "WRITE_SIZE"), is_copy)
    nbytes = copy_mb * 2 ** 20
    f_fac = cf * 1024 / nbytes
    w_fac = cw * 1024 / nbytes
    fetch = fk * 1024 / f_fac
    write = wk * 1024 / w_fac
    import kvq_synth as synth
    w = synth.WORKLOADS[workload]
    out = {"workload": workload, "decode_source_sha256": decode_source_sha(),
           "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk, "dispatches": [nf, nw],
           "copy_bytes": nbytes, "copy_fetch_factor": f_fac, "copy_write_factor": w_fac,
           "fetch_bytes": fetch, "write_bytes": write, "bytes_per_launch": fetch + write,
           "algorithmic_bytes_per_launch": decode_bytes(w)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama8b_8k")
    ap.add_argument("--rotate", type=int, default=0, help="cache copies to rotate over (0 = enough for >400 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", default="qwen32b_32k", help="extra decode-only workload ('' to skip)")
    ap.add_argument("--no-qjl", action="store_true", help="skip the QJL decodes (plain and outlier split)")
    ap.add_argument("--no-pnmix", action="store_true", help="skip the PN-Mix decode and flush")
    ap.add_argument("--no-fidelity", action="store_true", help="skip the per-workload fidelity (oracle, CPU)")
    ap.add_argument("--no-fifo", action="store_true", help="skip the Value-FIFO leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--decode-only", action="store_true", help="time the decode call only (for counter runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR", "MB"))
    return ap.parse_args()


class Rig:
    """Resident inputs for a workload, with `copies` rotated cache copies."""

    def __init__(self, w, copies, torch, kvq, synth, reselect=False):
        """reselect: MixKVQ with per-page records (the running query
        accumulator filled from the prefill queries, every prefill page
        flushed with its tiers re-selected)."""
        self.w, self.torch, self.kvq = w, torch, kvq
        dev = "cuda"
        self.g = w.group
        self.max_pages = w.n_pages + 1
        self.reselect = reselect
        self.cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, self.max_pages,
                                   n_bf16=w.n_bf16, n_u4=w.n_u4, n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m,
                                   page_records=1 if reselect else 0, qjl_outliers=w.qjl_outliers,
                                   qjl_m_out=w.qjl_m_out)
        pb = kvq.kvq_page_bytes(self.cfg)
        H = w.batch * w.n_kv_heads
        L = w.prefill_tokens
        q, k, v = synth.prefill(w, dev)
        self.S = synth.qjl_matrix(w, dev) if w.key_mode == 2 else None
        self.mask = torch.zeros(max(1, H * kvq.kvq_mask_bytes(self.cfg)), dtype=torch.uint8, device=dev)
        if reselect:
            self.acc = torch.zeros(H * 128 * 2, dtype=torch.int64, device=dev)
            kvq.kvq_accumulate_query(self.cfg, q, L, L, self.acc)
            self.mask = torch.zeros(H * self.max_pages * 160, dtype=torch.uint8, device=dev)
        elif w.key_mode == 0:
            kvq.kvq_select_channels(self.cfg, q, L, k.data_ptr() + w.n_sink * 256, w.n_pages * 128, self.mask,
                                    k_stride=L)
        elif w.key_mode == 1:
            kvq.kvq_select_channels(self.cfg, q, L, k, L, self.mask)
        elif w.qjl_outliers:   # QJL outlier channels from the prompt's Keys
            kvq.kvq_select_channels(self.cfg, None, 0, k, L, self.mask)
        del q
        arena = torch.zeros(H * self.max_pages * pb, dtype=torch.uint8, device=dev)
        self.flags = torch.zeros(4, dtype=torch.int32, device=dev)
        if reselect:
            kvq.kvq_flush_reselect(self.cfg, k, v, L, w.n_pages, self.acc, self.mask, arena, 0, self.flags)
        else:
            kvq.kvq_flush_quantize(self.cfg, k.data_ptr() + w.n_sink * 256, v.data_ptr() + w.n_sink * 256, L,
                                   w.n_pages, self.mask, self.S, arena, 0, self.flags)
        rk = torch.zeros(w.batch, w.n_kv_heads, 128, 128, dtype=torch.bfloat16, device=dev)
        rv = torch.zeros_like(rk)
        t0 = w.n_sink + w.n_pages * 128
        if w.n_resid:
            rk[:, :, :w.n_resid] = k[:, :, t0:t0 + w.n_resid]
            rv[:, :, :w.n_resid] = v[:, :, t0:t0 + w.n_resid]
        if w.n_resid < 128:   # the flush's source rows past the visible residual: the next tokens' K and V
            nk, nv = synth.appended_kv(w, 128, dev)
            rk[:, :, w.n_resid:] = nk[:, :, :128 - w.n_resid]
            rv[:, :, w.n_resid:] = nv[:, :, :128 - w.n_resid]
            del nk, nv
        self.sink_k = k[:, :, :w.n_sink].contiguous() if w.n_sink else None
        self.sink_v = v[:, :, :w.n_sink].contiguous() if w.n_sink else None
        del k, v
        self.arenas = [arena] + [arena.clone() for _ in range(copies - 1)]
        self.rks = [rk] + [rk.clone() for _ in range(copies - 1)]
        self.rvs = [rv] + [rv.clone() for _ in range(copies - 1)]
        self.q = synth.decode_query(w, dev)
        self.out = torch.zeros(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
        self.ws_bytes = kvq.kvq_workspace_bytes(self.cfg, w.n_pages)
        self.ws = torch.zeros(self.ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
        self.scale = 1.0 / math.sqrt(128)
        torch.cuda.synchronize()

    def decode(self, i):
        w = self.w
        c = i % len(self.arenas)
        self.kvq.kvq_decode_attention(self.cfg, self.q, self.arenas[c], w.n_pages, self.mask, self.S,
                                      self.sink_k, self.sink_v, w.n_sink, self.rks[c], self.rvs[c], w.n_resid,
                                      128, self.scale, self.out, self.ws, self.ws_bytes)

    def flush(self, i):
        w = self.w
        c = i % len(self.arenas)
        self.kvq.kvq_flush_quantize(self.cfg, self.rks[c], self.rvs[c], 128, 1, self.mask, self.S,
                                    self.arenas[c], w.n_pages, self.flags)

    def accumulate(self, i):
        self.kvq.kvq_accumulate_query(self.cfg, self.q, 1, 1, self.acc)

    def flush_reselect(self, i):
        w = self.w
        c = i % len(self.arenas)
        self.kvq.kvq_flush_reselect(self.cfg, self.rks[c], self.rvs[c], 128, 1, self.acc, self.mask,
                                    self.arenas[c], w.n_pages, self.flags)

    def make_paged(self, seed=7):
        """For every cache copy, the same pages scattered over the pool by a
        random permutation, and its page table."""
        torch, w = self.torch, self.w
        H = w.batch * w.n_kv_heads
        pool = H * self.max_pages
        gen = torch.Generator(device="cpu").manual_seed(seed)
        self.paged, self.tables = [], []
        for arena in self.arenas:
            perm = torch.randperm(pool, generator=gen).cuda()
            paged = torch.empty_like(arena)
            paged.view(pool, -1).index_copy_(0, perm, arena.view(pool, -1))
            self.paged.append(paged)
            self.tables.append(perm.to(torch.int32).reshape(H, self.max_pages))
        torch.cuda.synchronize()

    def decode_paged(self, i):
        w = self.w
        c = i % len(self.arenas)
        self.kvq.kvq_decode_attention(self.cfg, self.q, self.paged[c], w.n_pages, self.mask, self.S,
                                      self.sink_k, self.sink_v, w.n_sink, self.rks[c], self.rvs[c], w.n_resid,
                                      128, self.scale, self.out, self.ws, self.ws_bytes,
                                      page_table=self.tables[c], table_stride=self.max_pages)

    def decode_flush(self, i):
        """One step in one call: the decode, then the residual flushed into
        page n_pages, the flush sharing a launch with the decode's merge."""
        w = self.w
        c = i % len(self.arenas)
        self.kvq.kvq_decode_attention_flush(self.cfg, self.q, self.arenas[c], w.n_pages, self.mask, self.S,
                                            self.sink_k, self.sink_v, w.n_sink, self.rks[c], self.rvs[c],
                                            w.n_resid, 128, self.scale, self.out, self.ws, self.ws_bytes,
                                            self.rks[c], self.rvs[c], 128, 1, w.n_pages, self.flags)


def time_steps(rig, torch, steps, warmup, with_flush):
    """Eager calls, each bracketed by HIP events (used for counter runs)."""
    for i in range(warmup):
        rig.decode(i)
        if with_flush:
            rig.flush(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        a, b, c = ev[i]
        a.record()
        rig.decode(warmup + i)
        b.record()
        if with_flush:
            rig.flush(warmup + i)
        c.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec = [a.elapsed_time(b) for a, b, _ in ev]
    fl = [b.elapsed_time(c) for _, b, c in ev]
    return wall, dec, fl


def capture(torch, calls):
    """One HIP graph holding `calls` in order. The library launches on torch's
    current stream, which is the capture stream inside torch.cuda.graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for call in calls:
            call()
    torch.cuda.synchronize()
    return g


def replay_timed(torch, g):
    """(GPU ms from HIP events on the replay stream, host wall s) of one replay,
    bracketed by device synchronisation on both sides."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b), time.perf_counter() - t0


def graph_time(torch, calls, warmup_calls):
    """Per-call GPU ms of `calls` replayed as one graph, after one replay of a
    graph of `warmup_calls`."""
    if warmup_calls:
        capture(torch, warmup_calls).replay()
    g = capture(torch, calls)
    gpu_ms, wall = replay_timed(torch, g)
    del g
    return gpu_ms / len(calls), wall


def read_stream(torch, kvq, arenas, reps):
    """GB/s of a plain read of the same rotated cache copies by the library's
    read-stream reference (kvq_read_stream: the decode's load shape, one XOR
    word kept per 16 KB), timed like the decode. The read rate this GPU
    reaches at this size, which the decode's fraction of the 8 TB/s peak is
    to be read against."""
    nbytes = arenas[0].numel()
    sink = torch.zeros((nbytes + 16383) // 16384, dtype=torch.int32, device=arenas[0].device)
    call = lambda i: kvq.kvq_read_stream(arenas[i % len(arenas)], nbytes, sink, sink.numel() * 4)
    ms, _ = graph_time(torch, [lambda i=i: call(i) for i in range(reps)], [lambda i=i: call(i) for i in range(3)])
    return nbytes / (ms * 1e-3) / 1e9


def fifo_leg(w, copies, torch, kvq, synth, K, W):
    """KIVI's Value FIFO (blog sections 4-5) on the workload's shape in its
    steady state: n_pages sealed Key pages, 64 Key-residual rows, a 128-token
    full-precision Value window, every older Value quantized into its page.
    Times the FIFO decode (kvq_decode_attention_fifo) over rotated cache
    copies, the push of one Value row of every (batch, kv head)
    (kvq_value_push, distinct rows) and the seal of one Key page of every
    (batch, kv head) (kvq_flush_keys). The decode is timed on the default
    path (the pipelined kernel over every page and the Key residual, the
    merge adding the window Values of the tokens inside the pages) and on the
    generic path alone."""
    dev = "cuda"
    n_pages, n_kres, R = w.n_pages, 64, 128
    T = n_pages * 128 + n_kres
    n_vq = T - R
    H = w.batch * w.n_kv_heads
    L = w.prefill_tokens
    assert T <= L
    cfg = kvq.make_config(w.key_mode, w.batch, w.n_q_heads, w.n_kv_heads, n_pages + 1, n_bf16=w.n_bf16,
                          n_u4=w.n_u4, n_hi_pairs=w.n_hi_pairs, qjl_m=w.qjl_m)
    q, k, v = synth.prefill(w, dev)
    mask = torch.zeros(max(1, H * kvq.kvq_mask_bytes(cfg)), dtype=torch.uint8, device=dev)
    kvq.kvq_select_channels(cfg, q, L, k, n_pages * 128, mask, k_stride=L)
    del q
    arena = torch.zeros(H * (n_pages + 1) * kvq.kvq_page_bytes(cfg), dtype=torch.uint8, device=dev)
    flags = torch.zeros(4, dtype=torch.int32, device=dev)
    kvq.kvq_flush_keys(cfg, k, k, L, n_pages, mask, None, arena, 0, flags)
    kvq.kvq_value_push(cfg, v, L, n_vq, 0, mask, arena, flags)
    arenas = [arena] + [arena.clone() for _ in range(copies - 1)]
    row = 128 * 2
    kres, vwin = k.data_ptr() + n_pages * 128 * row, v.data_ptr() + n_vq * row
    qd = synth.decode_query(w, dev)
    out = torch.zeros(w.batch, w.n_q_heads, 128, dtype=torch.float32, device=dev)
    ws_bytes = kvq.kvq_workspace_bytes(cfg, n_pages)
    ws = torch.zeros(ws_bytes // 4 + 64, dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(128)

    cfg_generic = kvq.with_fields(cfg, decode_path=kvq.KVQ_DECODE_GENERIC)

    def dec(i, c=cfg):
        kvq.kvq_decode_attention_fifo(c, qd, arenas[i % copies], n_pages, n_vq, mask, None, kres, n_kres, L, vwin,
                                      R, L, scale, out, ws, ws_bytes)
    d_ms, _ = graph_time(torch, [lambda i=i: dec(i) for i in range(K)], [lambda i=i: dec(i) for i in range(W)])
    g_ms, _ = graph_time(torch, [lambda i=i: dec(i, cfg_generic) for i in range(K)],
                         [lambda i=i: dec(i, cfg_generic) for i in range(W)])
    # one Value row per call, rows n_vq, n_vq + 1, ... (not pushed before), into a scratch copy
    scratch = arenas[-1]
    n_push = min(K, R - n_kres)
    p_ms, _ = graph_time(torch, [lambda i=i: kvq.kvq_value_push(cfg, v.data_ptr() + (n_vq + i) * row, L, 1, n_vq + i,
                                                                 mask, scratch, flags) for i in range(n_push)], [])
    s_ms, _ = graph_time(torch, [lambda: kvq.kvq_flush_keys(cfg, kres, kres, L, 1, mask, None, scratch, n_pages,
                                                             flags)] * K, [])
    assert int(flags[0].item()) == 0
    per_head = n_pages * logical_page_bytes(w) + (n_kres + R) * row + record_bytes(w) + w.group * 128 * (2 + 4)
    dbytes = H * per_head
    gb = dbytes / (d_ms * 1e-3) / 1e9
    return {"workload": w.name, "sealed_pages": n_pages, "key_residual_tokens": n_kres, "quantized_values": n_vq,
            "value_window": R, "decode_ms": d_ms, "decode_GBps": gb, "decode_frac_hbm_peak": gb / HBM_PEAK_GBPS,
            "bytes_per_decode": dbytes,
            "decode_kernels": "decode_mix_fast<FIFO> (every page, Key residual; window-page logits) + "
                              "combine_fifo_kernel (merge + window Values)",
            "generic_path_ms": g_ms, "generic_path_GBps": dbytes / (g_ms * 1e-3) / 1e9,
            "value_push_ms": p_ms, "value_push_tokens_per_s": H / (p_ms * 1e-3),
            "key_seal_ms": s_ms, "key_seal_tokens_per_s": H * 128 / (s_ms * 1e-3)}


def fidelity(w, synth):
    """Fidelity context of the method on this data (not a parity gate), by the
    oracle alone on the slice (batch 0, kv head 0): KL(p_bf16 || p_quantized)
    of every query head of the group against exact attention over the
    unquantized bf16 cache of the same visible tokens, the quantized output's
    cosine and relative error, mean and worst over the heads."""
    import numpy as np
    from oracle import attention as oatt, flush as oflush, qjl as oqjl, select as osel
    w1 = w.scaled(batch=1)
    q, k, v = synth.prefill(w1, "cpu")
    bits = synth.bf16_bits
    g, h = w.group, 0
    qd = bits(synth.decode_query(w1, "cpu")[0, :g])
    kb, vb = bits(k[0, h]), bits(v[0, h])
    qb = bits(q[0, :g]) if w.key_mode != 2 else None
    del q
    ns, nq = w.n_sink, w.n_pages * 128
    kw = dict(scale=1 / math.sqrt(128))
    if w.key_mode == 0:
        tier, perm, _ = osel.mixkvq_select(qb, kb[ns:ns + nq], w.n_bf16, w.n_u4)
        pages = [oflush.flush_mixkvq_page(kb[ns + 128 * p:ns + 128 * p + 128], vb[ns + 128 * p:ns + 128 * p + 128],
                                          perm, w.n_bf16, w.n_u4) for p in range(w.n_pages)]
        extra = dict(n16=w.n_bf16, n4=w.n_u4, perm=perm)
    elif w.key_mode == 1:
        _, hi, rec = osel.pnmix_select(qb, kb, w.n_hi_pairs)
        pages = [oflush.flush_pnmix_page(kb[ns + 128 * p:ns + 128 * p + 128], vb[ns + 128 * p:ns + 128 * p + 128], hi)
                 for p in range(w.n_pages)]
        extra = dict(mask_rec=rec)
    else:
        S = bits(synth.qjl_matrix(w1, "cpu"))
        extra = dict(s_bits=S)
        if w.qjl_outliers:
            outl = oqjl.outlier_mask(kb, w.qjl_outliers)
            pages = [oflush.flush_qjl_page(kb[128 * p:128 * p + 128], vb[128 * p:128 * p + 128], S, m=w.qjl_m,
                                           outl=outl) for p in range(w.n_pages)]
            extra.update(qjl_m=w.qjl_m, outl=outl)
        else:
            pages = [oflush.flush_qjl_page(kb[128 * p:128 * p + 128], vb[128 * p:128 * p + 128], S)
                     for p in range(w.n_pages)]
    if ns:
        extra.update(sink_k=kb[:ns], sink_v=vb[:ns])
    if w.n_resid:
        extra.update(resid_k=kb[ns + nq:ns + nq + w.n_resid], resid_v=vb[ns + nq:ns + nq + w.n_resid])
    out_q, p_q = oatt.decode_arena_head(w.key_mode, qd, pages, kw["scale"], **extra)
    end = ns + nq + w.n_resid
    out_r, p_r = oatt.reference_attention(qd, kb[:end], vb[:end], kw["scale"])
    kl = [oatt.kl_divergence(a, b) for a, b in zip(p_r, p_q)]
    cos = np.sum(out_q * out_r, -1) / (np.linalg.norm(out_q, axis=-1) * np.linalg.norm(out_r, axis=-1))
    rel = np.max(np.abs(out_q - out_r), -1) / np.max(np.abs(out_r), -1)
    return {"slice": "batch 0, kv head 0", "visible_tokens": end, "kl_mean": float(np.mean(kl)),
            "kl_max": float(np.max(kl)), "cosine_mean": float(np.mean(cos)), "cosine_min": float(np.min(cos)),
            "out_rel_err_max": float(np.max(rel))}


def _cpu_worker(args):
    """One host process of the CPU baseline: the oracle on whole (batch, kv
    head) slices `heads` of the workload, single-threaded, until `budget_s`
    of its own time is spent (see cpu_baseline)."""
    name, heads, budget_s = args
    import kvq_synth as synth
    from threadpoolctl import threadpool_limits
    from oracle import attention as oatt, flush as oflush, select as osel
    w = synth.WORKLOADS[name]
    bmax = max(b for b, _ in heads)
    w1 = w.scaled(batch=bmax + 1)
    q, k, v = synth.prefill(w1, "cpu")
    bits = synth.bf16_bits
    g = w.group
    t_flush, n_flush, t_dec, n_dec = 0.0, 0, 0.0, 0
    built = []

    def decode(b, h, pages, perm, kb, vb, step):
        qd = synth.decode_query(w1, "cpu", step=step)
        t0 = time.perf_counter()
        oatt.decode_arena_head(0, bits(qd[b, h * g:(h + 1) * g]), pages, 1 / math.sqrt(128), n16=w.n_bf16,
                               n4=w.n_u4, perm=perm, resid_k=kb[w.n_pages * 128:], resid_v=vb[w.n_pages * 128:])
        return time.perf_counter() - t0

    with threadpool_limits(limits=1):
        for b, h in heads:
            qb, kb, vb = bits(q[b, h * g:(h + 1) * g]), bits(k[b, h]), bits(v[b, h])
            tier, perm, _ = osel.mixkvq_select(qb, kb[:w.n_pages * 128], w.n_bf16, w.n_u4)
            pages = []
            t0 = time.perf_counter()
            for p in range(w.n_pages):
                pages.append(oflush.flush_mixkvq_page(kb[128 * p:128 * p + 128], vb[128 * p:128 * p + 128],
                                                      perm, w.n_bf16, w.n_u4))
            t_flush += time.perf_counter() - t0
            n_flush += w.n_pages
            t_dec += decode(b, h, pages, perm, kb, vb, 0)
            n_dec += 1
            built.append((b, h, pages, perm, kb, vb))
            if t_flush + t_dec > budget_s:
                break
        step = 1
        while t_flush + t_dec <= budget_s:
            for b, h, pages, perm, kb, vb in built:
                t_dec += decode(b, h, pages, perm, kb, vb, step)
                n_dec += 1
                if t_flush + t_dec > budget_s:
                    break
            step += 1
    return t_flush, n_flush, t_dec, n_dec, len(built)


def host_cpu():
    """(usable cores, capped at the 16 a one-GPU machine's host share allows; CPU model)."""
    n = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return min(n, 16), n, model


def cpu_baseline_parallel(w, budget_s):
    """The oracle, as it stands, on the host's cores: one single-threaded
    process per core, each on its own whole (batch, kv head) slices of the
    workload (every page flush of the slice and its decode, then further
    decodes with the queries of later steps while its budget lasts). A step
    of a slice is one page flush plus one decode over all its pages and the
    residual, as on the GPU; the rate is the bytes of all the processes'
    flushes and decodes over the wall time."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor
    cores, avail, model = host_cpu()
    slices = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)][:cores]
    per = (decode_bytes(w) + flush_bytes(w)) / (w.batch * w.n_kv_heads)   # bytes of one slice step
    flush_b = flush_bytes(w) / (w.batch * w.n_kv_heads)
    dec_b = decode_bytes(w) / (w.batch * w.n_kv_heads)
    t0 = time.perf_counter()
    # fresh interpreters (spawn): forked copies of a process whose thread
    # pools are running can deadlock
    with ProcessPoolExecutor(max_workers=cores, mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(_cpu_worker, [(w.name, [bh], budget_s) for bh in slices]))
    wall = time.perf_counter() - t0
    n_flush = sum(r[1] for r in res)
    n_dec = sum(r[3] for r in res)
    busy = sum(r[0] + r[2] for r in res)
    total = n_flush * flush_b + n_dec * dec_b
    return {"value": total / busy * cores / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "host_cores_available": avail,
            "sample": f"{len(slices)} (batch, kv head) slices of {w.name}, one single-threaded oracle process per "
                      f"core: {n_flush} page flushes and {n_dec} decodes over {w.n_pages} pages + {w.n_resid} "
                      f"residual tokens, {budget_s:.0f} s of timed work per process ({wall:.1f} s wall with "
                      f"set-up); rate = algorithmic bytes of all of them / timed seconds per process",
            "step_s_per_slice": per / (total / busy) if total else None}


def cpu_tiny_one_thread(synth):
    """The oracle on the tiny MixKVQ workload, one thread: one decode over 8
    pages + 64 residual tokens, and one page flush, as s per step."""
    from threadpoolctl import threadpool_limits
    from oracle import attention as oatt, flush as oflush, select as osel
    w = synth.WORKLOADS["tiny_mixkvq"]
    q, k, v = synth.prefill(w, "cpu")
    bits = synth.bf16_bits
    qb, kb, vb = bits(q[0]), bits(k[0, 0]), bits(v[0, 0])
    qd = bits(synth.decode_query(w, "cpu")[0])
    with threadpool_limits(limits=1):
        tier, perm, _ = osel.mixkvq_select(qb, kb[:w.n_pages * 128], w.n_bf16, w.n_u4)
        t0 = time.perf_counter()
        pages = [oflush.flush_mixkvq_page(kb[128 * p:128 * p + 128], vb[128 * p:128 * p + 128], perm, w.n_bf16,
                                          w.n_u4) for p in range(w.n_pages)]
        t_fl = (time.perf_counter() - t0) / w.n_pages
        reps = 5
        t0 = time.perf_counter()
        for _ in range(reps):
            oatt.decode_arena_head(0, qd, pages, 1 / math.sqrt(128), n16=w.n_bf16, n4=w.n_u4, perm=perm,
                                   resid_k=kb[w.n_pages * 128:], resid_v=vb[w.n_pages * 128:])
        t_dec = (time.perf_counter() - t0) / reps
    return {"workload": w.name, "threads": 1, "flush_s_per_page": t_fl, "decode_s": t_dec,
            "step_GBps": (decode_bytes(w) + flush_bytes(w)) / (t_fl + t_dec) / 1e9}


def main():
    args = parse()
    if args.summarize_pmc:
        d = args.summarize_pmc
        summarize_pmc(d[0], d[1], d[2], d[3], int(d[4]), args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); multi-GPU sharding is "
              "described in DESIGN.md but not run", file=sys.stderr)
        sys.exit(2)
    # the CPU baseline runs first, in processes of its own, before this
    # process touches the GPU
    cpu = None
    if not (args.no_cpu_baseline or args.summarize_pmc or args.copy_calibration or args.decode_only):
        import kvq_synth as synth
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline_parallel(synth.WORKLOADS[args.workload], args.cpu_seconds)
        cpu["tiny_one_thread"] = cpu_tiny_one_thread(synth)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = args.copy_calibration * 2 ** 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}))
        return
    import kvq_synth as synth
    import mixed_precision_kv_amd as kvq
    kvq.load()

    w = synth.WORKLOADS[args.workload]
    cache_mb = decode_bytes(w) / 1e6
    copies = args.rotate or max(1, math.ceil(400.0 / cache_mb))
    print(f"[bench] {w.name}: {cache_mb:.1f} MB per decode, rotating {copies} copies", file=sys.stderr, flush=True)
    rig = Rig(w, copies, torch, kvq, synth)
    if args.decode_only:
        _, dec, _ = time_steps(rig, torch, args.steps, args.warmup, with_flush=False)
        print(json.dumps({"workload": w.name, "decode_ms": sum(dec) / len(dec)}))
        return
    K, W = args.steps, args.warmup
    dbytes, fbytes = decode_bytes(w), flush_bytes(w)

    def step(i):
        return [lambda i=i: rig.decode_flush(i)]

    # the timed region: K whole steps (decode + flush through
    # kvq_decode_attention_flush, rotating over the cache copies) replayed as
    # one HIP graph, so host launch cost stays outside
    warm_calls = [c for i in range(W) for c in step(i)]
    if warm_calls:
        capture(torch, warm_calls).replay()
    g_steps = capture(torch, [c for i in range(K) for c in step(W + i)])
    step_gpu_ms, wall = replay_timed(torch, g_steps)
    del g_steps
    ms_step = wall / K * 1e3
    # the dominant call (decode) and the flush on their own, same protocol
    dec_ms, _ = graph_time(torch, [lambda i=i: rig.decode(i) for i in range(K)],
                           [lambda i=i: rig.decode(i) for i in range(W)])
    fl_ms, _ = graph_time(torch, [lambda i=i: rig.flush(i) for i in range(K)], [])
    dec_gbps = dbytes / (dec_ms * 1e-3) / 1e9
    step_gbps = (dbytes + fbytes) / (ms_step * 1e-3) / 1e9
    flush_tok_s = w.batch * 128 / (fl_ms * 1e-3)
    # warm-cache decode (no rotation) as a secondary number
    dec_w_ms, _ = graph_time(torch, [lambda: rig.decode(0)] * K, [lambda: rig.decode(0)] * 3)
    dec_warm_gbps = dbytes / (dec_w_ms * 1e-3) / 1e9
    rs_gbps = read_stream(torch, kvq, rig.arenas, K)
    # the same decode with its pages scattered over the pool (page table)
    rig.make_paged()
    dec_p_ms, _ = graph_time(torch, [lambda i=i: rig.decode_paged(i) for i in range(K)],
                             [lambda i=i: rig.decode_paged(i) for i in range(W)])
    del rig
    torch.cuda.empty_cache()

    extra = {}
    if args.secondary:
        w2 = synth.WORKLOADS[args.secondary]
        mb2 = decode_bytes(w2) / 1e6
        print(f"[bench] secondary {w2.name}: {mb2:.1f} MB per decode", file=sys.stderr, flush=True)
        rig2 = Rig(w2, max(1, math.ceil(400.0 / mb2)), torch, kvq, synth)
        k2 = max(10, K // 2)
        d2, _ = graph_time(torch, [lambda i=i: rig2.decode(i) for i in range(k2)],
                           [lambda i=i: rig2.decode(i) for i in range(3)])
        rs2 = read_stream(torch, kvq, rig2.arenas, k2)
        rig2.make_paged()
        d2p, _ = graph_time(torch, [lambda i=i: rig2.decode_paged(i) for i in range(k2)],
                            [lambda i=i: rig2.decode_paged(i) for i in range(3)])
        gb2 = decode_bytes(w2) / (d2 * 1e-3) / 1e9
        extra = {"workload": w2.name, "decode_ms": d2, "decode_GBps": gb2,
                 "decode_frac_hbm_peak": gb2 / HBM_PEAK_GBPS, "read_stream_GBps": rs2,
                 "decode_frac_read_stream": gb2 / rs2,
                 "decode_paged_ms": d2p, "decode_paged_GBps": decode_bytes(w2) / (d2p * 1e-3) / 1e9}
        del rig2
        torch.cuda.empty_cache()

    # PN-Mix H3/L1 (32 sinks + 16K quantized + 128 residual, batch 32): the
    # decode over rotated cache copies and the flush of the residual
    pnmix = {}
    if not args.no_pnmix:
        wp = synth.WORKLOADS["pnmix_16k"]
        mbp = decode_bytes(wp) / 1e6
        print(f"[bench] pnmix_16k: {mbp:.1f} MB per decode", file=sys.stderr, flush=True)
        rp = Rig(wp, max(1, math.ceil(400.0 / mbp)), torch, kvq, synth)
        kp = max(10, K // 2)
        dp, _ = graph_time(torch, [lambda i=i: rp.decode(i) for i in range(kp)],
                           [lambda i=i: rp.decode(i) for i in range(3)])
        fp, _ = graph_time(torch, [lambda i=i: rp.flush(i) for i in range(kp)], [])
        rsp = read_stream(torch, kvq, rp.arenas, kp)
        gb = decode_bytes(wp) / (dp * 1e-3) / 1e9
        pnmix = {"workload": wp.name, "decode_ms": dp, "decode_GBps": gb, "decode_frac_hbm_peak": gb / HBM_PEAK_GBPS,
                 "read_stream_GBps": rsp, "decode_frac_read_stream": gb / rsp,
                 "bytes_per_decode": decode_bytes(wp), "cache_copies_rotated": len(rp.arenas),
                 "flush_ms": fp, "flush_tokens_per_s": wp.batch * 128 / (fp * 1e-3),
                 "flush_GBps": flush_bytes(wp) / (fp * 1e-3) / 1e9}
        del rp
        torch.cuda.empty_cache()

    # QJL at 32K context: the plain sketch and the outlier split (two sketch
    # instances), decode calls over the resident cache and the sketch flush
    # of 128 new tokens
    qjl = {}
    if not args.no_qjl:
        for name in ("qjl_32k", "qjl_outlier_32k"):
            wq = synth.WORKLOADS[name]
            print(f"[bench] {name}: {decode_bytes(wq) / 1e6:.1f} MB per decode", file=sys.stderr, flush=True)
            rq = Rig(wq, 1, torch, kvq, synth)
            kq = max(10, K // 2)
            dq, _ = graph_time(torch, [lambda: rq.decode(0)] * kq, [lambda: rq.decode(0)] * 3)
            fq, _ = graph_time(torch, [lambda: rq.flush(0)] * kq, [])
            rsq = read_stream(torch, kvq, rq.arenas, kq)
            gb = decode_bytes(wq) / (dq * 1e-3) / 1e9
            qjl[name] = {"decode_ms": dq, "decode_GBps": gb, "decode_frac_hbm_peak": gb / HBM_PEAK_GBPS,
                         "read_stream_GBps": rsq, "decode_frac_read_stream": gb / rsq,
                         "bytes_per_decode": decode_bytes(wq), "page_bytes_logical": logical_page_bytes(wq),
                         "flush_ms": fq, "flush_tokens_per_s": wq.batch * 128 / (fq * 1e-3),
                         "flush_GBps": flush_bytes(wq) / (fq * 1e-3) / 1e9}
            del rq
            torch.cuda.empty_cache()

    # per-flush reselection (MixKVQ's running query accumulator; per-page
    # records read by the decode): the decode, the accumulation of the step's
    # query, the reselecting one-page flush, and the step of all three
    resel = {}
    if w.key_mode == 0:
        rr = Rig(w, copies, torch, kvq, synth, reselect=True)
        kr = max(10, K // 2)
        r_dec, _ = graph_time(torch, [lambda i=i: rr.decode(i) for i in range(kr)], [lambda i=i: rr.decode(i) for i in range(3)])
        r_acc, _ = graph_time(torch, [lambda i=i: rr.accumulate(i) for i in range(kr)], [])
        r_fl, _ = graph_time(torch, [lambda i=i: rr.flush_reselect(i) for i in range(kr)], [])
        steps_r = [c for i in range(kr) for c in (lambda i=i: rr.accumulate(i), lambda i=i: rr.decode(i),
                                                  lambda i=i: rr.flush_reselect(i))]
        r_step, _ = graph_time(torch, steps_r, [])
        r_step *= 3   # graph_time divides by the number of calls
        resel = {"decode_ms": r_dec, "accumulate_ms": r_acc, "flush_reselect_ms": r_fl, "step_ms": r_step,
                 "decode_GBps": dbytes / (r_dec * 1e-3) / 1e9,
                 "step_GBps": (dbytes + fbytes) / (r_step * 1e-3) / 1e9}
        del rr
        torch.cuda.empty_cache()


    # KIVI's Value FIFO in its steady state on the same shape
    fifo = {}
    if w.key_mode == 0 and not args.no_fifo:
        print(f"[bench] value FIFO on {w.name}", file=sys.stderr, flush=True)
        fifo = fifo_leg(w, copies, torch, kvq, synth, max(10, K // 2), 3)
        torch.cuda.empty_cache()

    fid = {}
    if not args.no_fidelity:
        for name in ("llama8b_8k", "qwen32b_32k", "pnmix_16k", "qjl_32k", "qjl_outlier_32k"):
            print(f"[bench] fidelity {name} (oracle)", file=sys.stderr, flush=True)
            fid[name] = fidelity(synth.WORKLOADS[name], synth)

    line = {
        "metric": METRIC,
        "value": step_gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_gpu_ms": step_gpu_ms / K,
        "step_call": "kvq_decode_attention_flush (decode kernel; flush blocks + split merge in one launch)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "quantized_tokens": w.n_pages * 128, "residual_tokens": w.n_resid,
                   "key_tiers_bf16_u4_u2": [w.n_bf16, w.n_u4, 128 - w.n_bf16 - w.n_u4],
                   "cache_copies_rotated": copies},
        "decode_GBps": dec_gbps,
        "decode_frac_hbm_peak": dec_gbps / HBM_PEAK_GBPS,
        "decode_ms": dec_ms,
        "decode_warm_GBps": dec_warm_gbps,
        "read_stream_GBps": rs_gbps,
        "decode_frac_read_stream": dec_gbps / rs_gbps,
        "decode_paged_ms": dec_p_ms,
        "decode_paged_GBps": dbytes / (dec_p_ms * 1e-3) / 1e9,
        "flush_tokens_per_s": flush_tok_s,
        "flush_ms": fl_ms,
        "roofline": {"bound": "hbm", "achieved": dec_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": dec_gbps / HBM_PEAK_GBPS, "traffic": committed_traffic(w.name),
                     "kernel": "kvq_decode_attention (decode_mix_fast + combine_kernel)",
                     "bytes_per_launch": dbytes},
        "secondary": extra,
        "pnmix": pnmix,
        "reselect_per_flush": resel,
        "value_fifo": fifo,
        "qjl_decode": qjl,
        "fidelity": fid,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
