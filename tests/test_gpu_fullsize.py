"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (same config, page count, batch and workspace).

The whole cache is built on the GPU; the oracle recomputes sampled
(batch, kv head) slices from its own selection records: the record and every
page of the slice bit-exact, the decode output of the slice's query heads
within the 2e-3 relative bound, and the benchmark's one-page flush of the
residual into page n_pages bit-exact. At these sizes every split of the
decode covers several pages (4 for llama8b_8k, 16 or more for the others), so the
multi-page paths the benchmark times are the ones checked:

* the pipelined kernel over the contiguous cache (the benchmark's call);
* the generic kernel (decode_path KVQ_DECODE_GENERIC) over the same cache;
* both kernels with the pages scattered over the pool by a random
  permutation and reached through a page table (the benchmark's paged
  decode): bit-identical to the contiguous runs, which are checked against
  the oracle on the sampled slices.

On every query head (not only the sampled ones) the two kernels, which share
no page-loop code, agree within twice the bound, and every output is finite.
"""
import numpy as np
import pytest
import torch

import kvq_synth as synth
import mixed_precision_kv_amd as kvq
from kvq_harness import Pipeline, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU"),
              pytest.mark.timeout(900)]

TOL = 2e-3
NAMES = ["llama8b_8k", "qwen32b_32k", "pnmix_16k", "qjl_32k", "qjl_outlier_32k"]


def slices(w):
    """Sampled (batch, kv head) slices: corners and a few in between (a QJL
    page costs the oracle ~0.2 s, so two slices of 256 pages there)."""
    last = (w.batch - 1, w.n_kv_heads - 1)
    if w.key_mode == synth.QJL:
        return [last, (w.batch // 2, 3)]
    mid = [(w.batch // 2, w.n_kv_heads // 2), (1, w.n_kv_heads - 2)]
    if w.name == "llama8b_8k":
        mid += [(3, 1), (6, 6)]
    return [(0, 0), last] + mid


def oracle_pages(p, b, h):
    """The oracle's pages of slice (b, h) under the oracle's own record,
    cached per slice."""
    cache = p.__dict__.setdefault("_oracle_pages", {})
    if (b, h) not in cache:
        rec = p.oracle_recs[(b, h)]
        cache[(b, h)] = [p.oracle_page(b, h, pg, rec) for pg in range(p.w.n_pages)]
    return cache[(b, h)]


def paged(p, seed):
    """The arena's pages scattered over the pool by a random permutation, and
    the page table that reaches them."""
    w = p.w
    heads = w.batch * w.n_kv_heads
    pool = heads * p.max_pages
    gen = torch.Generator(device="cpu").manual_seed(seed)
    perm = torch.randperm(pool, generator=gen).cuda()
    arena2 = torch.empty_like(p.arena)
    arena2.view(pool, -1).index_copy_(0, perm, p.arena.view(pool, -1))
    return arena2, perm.to(torch.int32).reshape(heads, p.max_pages)


def decode_call(p, cfg, arena, out, table=None):
    w = p.w
    kvq.kvq_decode_attention(cfg, p.q_dec, arena, w.n_pages, p.mask, p.S, p.sink_k, p.sink_v, w.n_sink, p.resid_k,
                             p.resid_v, w.n_resid, 128, p.scale, out, p.ws, p.ws_bytes, page_table=table,
                             table_stride=p.max_pages if table is not None else 0)


@pytest.fixture(scope="module", params=NAMES)
def full(request):
    w = synth.WORKLOADS[request.param]
    print(f"\n[case] full size {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    # the oracle's records of the sampled slices, while the prefill queries are resident
    p.oracle_recs = {bh: (p.oracle_record(*bh) if p.mask_bytes else None) for bh in slices(w)}
    p.q_pre = None
    torch.cuda.empty_cache()
    outs = {}
    generic_cfg = kvq.with_fields(p.cfg, decode_path=kvq.KVQ_DECODE_GENERIC)
    for tag, cfg in (("fast", p.cfg), ("generic", generic_cfg)):
        outs[tag] = torch.zeros_like(p.out)
        decode_call(p, cfg, p.arena, outs[tag])
    arena2, table = paged(p, 97 + w.seed)
    for tag, cfg in (("fast_paged", p.cfg), ("generic_paged", generic_cfg)):
        outs[tag] = torch.zeros_like(p.out)
        decode_call(p, cfg, arena2, outs[tag], table)
    torch.cuda.synchronize()
    del arena2, table
    # the benchmark's flush: the 128-token residual buffer into page n_pages
    kvq.kvq_flush_quantize(p.cfg, p.resid_k, p.resid_v, 128, 1, p.mask, p.S, p.arena, w.n_pages, p.flags)
    torch.cuda.synchronize()
    yield request.param, p, {k: v.cpu().numpy() for k, v in outs.items()}
    del p
    torch.cuda.empty_cache()


def test_fullsize_records(full):
    name, p, _ = full
    if not p.mask_bytes:
        pytest.skip("plain QJL has no selection")
    for b, h in slices(p.w):
        assert np.array_equal(p.gpu_record(b, h), p.oracle_recs[(b, h)]), (name, b, h)


def test_fullsize_select_and_pages(full):
    name, p, _ = full
    assert int(p.flags[0].item()) == 0
    for b, h in slices(p.w):
        print(f"[pages] {name} b{b} h{h}", flush=True)
        for pg, ref in enumerate(oracle_pages(p, b, h)):
            assert p.same_page(p.gpu_page(b, h, pg), ref), (name, b, h, pg)


def test_fullsize_decode(full):
    """Both kernels, contiguous and through a page table, against the oracle."""
    name, p, outs = full
    w = p.w
    g = p.g
    assert np.array_equal(outs["fast_paged"], outs["fast"])
    assert np.array_equal(outs["generic_paged"], outs["generic"])
    for o in outs.values():
        assert np.all(np.isfinite(o))
    for b, h in slices(w):
        print(f"[decode] {name} b{b} h{h}", flush=True)
        ref, _ = p.oracle_decode(b, h, oracle_pages(p, b, h), p.oracle_recs[(b, h)])
        for tag in ("fast", "generic"):
            err = rel_err(outs[tag][b, h * g:(h + 1) * g], ref)
            print(f"[decode] {name} {tag} b{b} h{h}: worst relative error {err.max():.3e}")
            assert np.all(err <= TOL), (name, tag, b, h, err)
    # every query head: the two kernels agree
    both = rel_err(outs["fast"].reshape(-1, 128), outs["generic"].reshape(-1, 128))
    print(f"[decode] {name}: fast vs generic over {both.size} heads, worst {both.max():.3e}")
    assert np.all(both <= 2 * TOL)


def test_fullsize_residual_flush(full):
    name, p, _ = full
    w = p.w
    for b, h in slices(w):
        kb, vb = p.bits(p.resid_k[b, h]), p.bits(p.resid_v[b, h])
        ref = p.oracle_flush(kb, vb, p.oracle_recs[(b, h)])
        assert p.same_page(p.gpu_page(b, h, w.n_pages), ref), (name, b, h)


def test_fullsize_fidelity(full):
    """Fidelity context (not a parity gate): against attention on the
    unquantized bf16 cache of the same visible tokens, the mean KL(p_bf16 ||
    p_quantized) over the slice's query heads (the oracle's probabilities on
    the dequantized cache), and the GPU output's relative error and cosine.

    The synthetic K and V are Gaussian (plus the outlier channels), the
    hardest case for 2-bit codes: with 115 UINT2 Key channels the score
    noise alone predicts a KL near 0.1, so the bounds are only sanity checks
    that catch a broken path (wrong tokens, scale or order)."""
    from oracle import attention as oatt
    name, p, outs = full
    w = p.w
    b, h = slices(w)[0]
    rec = p.oracle_recs[(b, h)]
    _, probs_q = p.oracle_decode(b, h, oracle_pages(p, b, h), rec)
    out_r, probs_r = p.reference_probs(b, h, w.n_pages, w.n_resid)
    kl = float(np.mean([oatt.kl_divergence(pr, pq) for pr, pq in zip(probs_r, probs_q)]))
    o = outs["fast"][b, h * p.g:(h + 1) * p.g].astype(np.float64)
    rel = float(np.max(rel_err(o, out_r)))
    cos = float(np.min(np.sum(o * out_r, -1) / (np.linalg.norm(o, axis=-1) * np.linalg.norm(out_r, axis=-1))))
    print(f"[fidelity] {name} b{b} h{h}: KL {kl:.3e}, output rel err {rel:.3e}, cosine {cos:.5f}")
    assert np.isfinite(kl) and kl < 1.0 and cos > 0.5, (name, kl, cos)
