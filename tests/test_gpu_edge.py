"""GPU edge cases of libkvq against the oracle.

* The generic decode kernel (decode_path KVQ_DECODE_GENERIC) against the oracle
  and against the pipelined kernels.
* Degenerate visible sets: no pages, only residual; no pages and no
  residual; a prefix of the flushed pages.
* The tiny MixKVQ flow of the workload list: decode over 8 pages + 64
  residual tokens, append 64 tokens, flush the full residual into page 8
  (bit-exact), decode again over 9 pages.
* Flush status flags: non-finite inputs, values beyond the binary16 range,
  groups spanning more than 38 binades; constant groups bit-exact. The
  non-finite flag for an element in any part of a group's scan (MixKVQ and
  PN-Mix); an infinite Value element leaves every other group of its page
  as the oracle's.
* A page flagged KVQ_FLAG_RANGE (infinite binary16 metadata) decodes to
  non-finite outputs for its own (batch, kv head)'s query heads only.
* PN-Mix with the adjacent pair layout; a PN-Mix record with another pair
  count raises KVQ_FLAG_MASK.
* Repeated decode calls give identical bits.
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


def check_decode(p, n_pages, n_resid, tag):
    out = p.out.cpu().numpy()
    g = p.g
    for b in range(p.w.batch):
        for h in range(p.w.n_kv_heads):
            rec = p.record(b, h)
            pages = [p.oracle_page(b, h, pg, rec) for pg in range(n_pages)]
            ref, _ = p.oracle_decode(b, h, pages, rec, n_resid=n_resid)
            err = rel_err(out[b, h * g:(h + 1) * g], ref)
            assert np.all(err <= TOL), (tag, b, h, err)


def built(w, **kw):
    print(f"\n[case] {w}", flush=True)
    p = Pipeline(w, **kw)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    return p


@pytest.mark.parametrize("name", ["llama8b_8k", "qwen32b_32k", "pnmix_16k", "qjl_32k", "qjl_outlier_32k"])
def test_generic_decode_matches_oracle_and_fast(name):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=1, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=3, n_resid=min(base.n_resid, 40),
                    seed=base.seed + 100)
    p = built(w)
    p.decode(generic=True)
    torch.cuda.synchronize()
    generic = p.out.clone()
    check_decode(p, w.n_pages, w.n_resid, name + "/generic")
    p.decode()
    torch.cuda.synchronize()
    fast = p.out.clone()
    check_decode(p, w.n_pages, w.n_resid, name + "/fast")
    ref = generic.cpu().numpy().reshape(-1, 128)
    assert np.all(rel_err(fast.cpu().numpy().reshape(-1, 128), ref) <= 2 * TOL)


@pytest.mark.parametrize("name", ["llama8b_8k", "pnmix_16k", "qjl_32k"])
def test_degenerate_visible_sets(name):
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=2, n_kv_heads=1, n_q_heads=base.group, n_pages=4, n_resid=60, seed=base.seed + 200)
    p = built(w)
    # no pages: sinks (PN-Mix) + residual only
    p.decode(n_pages=0, n_resid=60)
    torch.cuda.synchronize()
    check_decode(p, 0, 60, name + "/no-pages")
    # a prefix of the flushed pages, no residual
    p.decode(n_pages=2, n_resid=0)
    torch.cuda.synchronize()
    check_decode(p, 2, 0, name + "/prefix")
    # nothing visible (no sinks either): every output is zero
    if w.n_sink == 0:
        p.out.fill_(7.0)
        p.decode(n_pages=0, n_resid=0)
        torch.cuda.synchronize()
        assert torch.count_nonzero(p.out).item() == 0


def test_tiny_decode_append_flush_decode():
    w = synth.WORKLOADS["tiny_mixkvq"]
    p = built(w)
    assert int(p.flags[0].item()) == 0
    p.decode()
    torch.cuda.synchronize()
    check_decode(p, w.n_pages, w.n_resid, "tiny/first decode")
    # 64 more seeded tokens fill the residual to 128, which is flushed into page 8
    k_new, v_new = synth.appended_kv(w, w.n_append, "cuda")
    p.resid_k[:, :, w.n_resid:w.n_resid + w.n_append] = k_new
    p.resid_v[:, :, w.n_resid:w.n_resid + w.n_append] = v_new
    kvq.kvq_flush_quantize(p.cfg, p.resid_k, p.resid_v, 128, 1, p.mask, None, p.arena, w.n_pages, p.flags)
    torch.cuda.synchronize()
    assert int(p.flags[0].item()) == 0
    rec = p.gpu_record(0, 0)
    from oracle import flush as oflush
    ref = oflush.flush_mixkvq_page(p.bits(p.resid_k[0, 0]), p.bits(p.resid_v[0, 0]), rec[:128], w.n_bf16, w.n_u4)
    assert np.array_equal(p.gpu_page(0, 0, w.n_pages), ref)
    # decode over the 9 pages, empty residual
    p.decode(n_pages=w.n_pages + 1, n_resid=0)
    torch.cuda.synchronize()
    out = p.out.cpu().numpy()
    pages = [p.oracle_page(0, 0, pg, rec) for pg in range(w.n_pages)] + [ref]
    refo, _ = p.oracle_decode(0, 0, pages, rec, n_resid=0)
    assert np.all(rel_err(out[0, :w.group], refo) <= TOL)


def _flush_one(p, k, v):
    """Flush one page from explicit [B, Hkv, 128, D] K / V into page 0."""
    p.flags.zero_()
    kvq.kvq_flush_quantize(p.cfg, k, v, 128, 1, p.mask, p.S, p.arena, 0, p.flags)
    torch.cuda.synchronize()
    return int(p.flags[0].item())


def test_flush_constant_groups_and_flags():
    w = synth.WORKLOADS["tiny_mixkvq"].scaled(n_pages=1, n_resid=0, n_append=0, seed=1301)
    p = built(w)
    rec = p.gpu_record(0, 0)
    from oracle import flush as oflush
    k = p.k_pre[:, :, :128].clone()
    v = p.v_pre[:, :, :128].clone()
    # constant Key channels (every tier) and constant value groups: bit-exact, no flag
    for d in (int(rec[0]), int(rec[20]), int(rec[100]), 5):
        k[0, 0, :, d] = 1.5
    v[0, 0, 3, 0:32] = -2.25
    v[0, 0, 7, :] = 0.0
    assert _flush_one(p, k, v) == 0
    ref = oflush.flush_mixkvq_page(p.bits(k[0, 0]), p.bits(v[0, 0]), rec[:128], w.n_bf16, w.n_u4)
    assert np.array_equal(p.gpu_page(0, 0, 0), ref)
    # beyond the binary16 range: infinite scale / offset, KVQ_FLAG_RANGE, still bit-exact
    k2 = k.clone()
    k2[0, 0, 10, int(rec[100])] = 4.0e5
    v2 = v.clone()
    v2[0, 0, 9, 40] = -3.0e5
    f = _flush_one(p, k2, v2)
    assert f & kvq.KVQ_FLAG_RANGE and not f & (kvq.KVQ_FLAG_NONFINITE | kvq.KVQ_FLAG_SPAN), f
    ref = oflush.flush_mixkvq_page(p.bits(k2[0, 0]), p.bits(v2[0, 0]), rec[:128], w.n_bf16, w.n_u4)
    assert np.array_equal(p.gpu_page(0, 0, 0), ref)
    # a value group spanning more than 38 binades: KVQ_FLAG_SPAN
    v3 = v.clone()
    v3[0, 0, 11, 64] = 2.0 ** -60
    v3[0, 0, 11, 65] = 2.0 ** 20
    assert _flush_one(p, k, v3) & kvq.KVQ_FLAG_SPAN
    # a non-finite input: KVQ_FLAG_NONFINITE
    v4 = v.clone()
    v4[0, 0, 2, 2] = float("nan")
    assert _flush_one(p, k, v4) & kvq.KVQ_FLAG_NONFINITE
    k5 = k.clone()
    k5[0, 0, 4, int(rec[0])] = float("inf")          # a BF16-tier channel
    assert _flush_one(p, k5, v) & kvq.KVQ_FLAG_NONFINITE


def test_flush_infinite_value_stays_in_its_group():
    """An infinite Value element: KVQ_FLAG_NONFINITE, its group's codes are
    unspecified, and every other code, scale and offset of the page is the
    oracle's. The group's bits are those that change when the element is
    replaced by finite values far above, far below and inside the group's
    range (widened to whole 16-bit halves, so that the group's scale and
    offset are free too). The element sits in an even token, whose codes
    share their 32-bit words with the next token's: a code that is not cut to
    its 2-bit field reaches them."""
    from oracle import flush as oflush
    w = synth.WORKLOADS["tiny_mixkvq"].scaled(n_pages=1, n_resid=0, n_append=0, seed=1305)
    p = built(w)
    rec = p.gpu_record(0, 0)
    k = p.k_pre[:, :, :128].clone()
    v = p.v_pre[:, :, :128].clone()
    for tok, ch in ((4, 37), (66, 0), (34, 20), (120, 127)):
        v_inf = v.clone()
        v_inf[0, 0, tok, ch] = float("inf")
        f = _flush_one(p, k, v_inf)
        assert f & kvq.KVQ_FLAG_NONFINITE, (tok, ch, f)
        gpu = p.gpu_page(0, 0, 0)
        refs = []
        for sub in (1.0e4, -1.0e4, 0.0):
            v_sub = v.clone()
            v_sub[0, 0, tok, ch] = sub
            refs.append(oflush.flush_mixkvq_page(p.bits(k[0, 0]), p.bits(v_sub[0, 0]), rec[:128], w.n_bf16, w.n_u4))
        free = np.zeros_like(refs[0])
        for r in refs[1:]:
            free |= refs[0] ^ r
        pairs = free.reshape(-1, 2).any(axis=1)
        free = np.repeat(np.where(pairs, 0xFF, 0), 2).astype(np.uint8)
        assert 0 < np.count_nonzero(free) < 64, (tok, ch)
        got = np.asarray(gpu)[:refs[0].size]
        assert np.array_equal(got & ~free, refs[0] & ~free), (tok, ch)


@pytest.mark.parametrize("name", ["tiny_mixkvq", "pnmix_16k"])
def test_flush_nonfinite_flag_at_every_position(name):
    """KVQ_FLAG_NONFINITE for one infinite or NaN Key or Value element, wherever
    it sits: a group's minimum, maximum and status are reduced over the
    threads that scan parts of it (two per value group and PN-Mix Key slot,
    eight per MixKVQ Key slot), and the flag of every part reaches the
    thread that reports it."""
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=1, n_kv_heads=1, n_q_heads=base.group, n_pages=1, n_resid=0, n_append=0,
                    seed=base.seed + 1307)
    p = built(w)
    k = p.k_pre[:, :, :128].clone()
    v = p.v_pre[:, :, :128].clone()
    assert _flush_one(p, k, v) == 0
    for val in (float("inf"), float("-inf"), float("nan")):
        for tok in (0, 17, 63, 64, 100, 127):
            for ch in (0, 16, 31, 45, 112, 127):
                for which in ("k", "v"):
                    kk, vv = k.clone(), v.clone()
                    (kk if which == "k" else vv)[0, 0, tok, ch] = val
                    f = _flush_one(p, kk, vv)
                    assert f & kvq.KVQ_FLAG_NONFINITE, (name, which, val, tok, ch, f)


def test_pnmix_record_pair_count_flag():
    """A PN-Mix record that selects another pair count than n_hi_pairs (one
    pair more, one fewer) raises KVQ_FLAG_MASK; the selection's own record
    raises nothing."""
    base = synth.WORKLOADS["pnmix_16k"]
    w = base.scaled(batch=1, n_kv_heads=1, n_q_heads=base.group, n_pages=1, n_resid=0, n_append=0,
                    seed=base.seed + 1309)
    p = built(w)
    k = p.k_pre[:, :, :128].clone()
    v = p.v_pre[:, :, :128].clone()
    assert _flush_one(p, k, v) == 0
    own = p.mask[:8].clone()
    pm = int.from_bytes(bytes(own.cpu().numpy().tolist()), "little")
    assert bin(pm).count("1") == w.n_hi_pairs
    unset = next(i for i in range(64) if not (pm >> i) & 1)
    first = next(i for i in range(64) if (pm >> i) & 1)
    for other in (pm | (1 << unset), pm & ~(1 << first)):
        p.mask[:8] = torch.tensor(list(other.to_bytes(8, "little")), dtype=torch.uint8, device="cuda")
        assert _flush_one(p, k, v) & kvq.KVQ_FLAG_MASK, hex(other)
    p.mask[:8] = own
    assert _flush_one(p, k, v) == 0


def test_pnmix_adjacent_pairs():
    base = synth.WORKLOADS["pnmix_16k"]
    w = base.scaled(batch=1, n_kv_heads=2, n_q_heads=8, n_pages=2, n_resid=33, seed=1401)
    p = built(w, pair_layout="adjacent")
    for h in range(w.n_kv_heads):
        assert np.array_equal(p.gpu_record(0, h), p.oracle_record(0, h))
        for pg in range(w.n_pages):
            assert np.array_equal(p.gpu_page(0, h, pg), p.oracle_page(0, h, pg, p.gpu_record(0, h)))
    p.decode()
    torch.cuda.synchronize()
    check_decode(p, w.n_pages, w.n_resid, "pnmix/adjacent")


def test_decode_is_deterministic():
    w = synth.WORKLOADS["llama8b_8k"].scaled(batch=2, n_pages=6, seed=1501)
    p = built(w)
    p.decode()
    torch.cuda.synchronize()
    first = p.out.clone()
    for _ in range(3):
        p.decode()
    torch.cuda.synchronize()
    assert torch.equal(first, p.out)


@pytest.mark.parametrize("name", ["tiny_mixkvq", "pnmix_16k", "qjl_32k"])
def test_flush_ties_bit_exact(name):
    """Integer-valued K and V on 0..6 (and 0..30 in the UINT4 channels): many
    codes fall exactly on a rounding midpoint, and PN-Mix values on the 1-bit
    midpoint, so the tie-breaking path of every quantizer is exercised."""
    base = synth.WORKLOADS[name]
    w = base.scaled(batch=1, n_kv_heads=2, n_q_heads=2 * base.group, n_pages=2, n_resid=0, n_append=0,
                    seed=base.seed + 500)
    p = built(w)
    gen = torch.Generator(device="cpu").manual_seed(77)
    k = torch.randint(0, 7, (1, 2, 128, 128), generator=gen).to(torch.bfloat16)
    v = torch.randint(0, 7, (1, 2, 128, 128), generator=gen).to(torch.bfloat16)
    k[..., ::5] *= 5                                       # some channels on 0..30
    k, v = k.cuda(), v.cuda()
    assert _flush_one(p, k, v) == 0
    from oracle import flush as oflush
    from oracle import select as osel
    for h in range(2):
        kb, vb = p.bits(k[0, h]), p.bits(v[0, h])
        if w.key_mode == synth.MIXKVQ:
            ref = oflush.flush_mixkvq_page(kb, vb, p.gpu_record(0, h)[:128], w.n_bf16, w.n_u4)
        elif w.key_mode == synth.PNMIX:
            ref = oflush.flush_pnmix_page(kb, vb, osel.hi_channels_from_record(p.gpu_record(0, h)))
        else:
            ref = oflush.flush_qjl_page(kb, vb, p.bits(p.S))
        assert np.array_equal(p.gpu_page(0, h, 0), ref), (name, h)


@pytest.mark.parametrize("part", ["key", "value"])
def test_range_flagged_page_decodes_non_finite(part):
    """The decode over a page whose flush stored an infinite binary16 scale or
    offset (KVQ_FLAG_RANGE) gives non-finite outputs for every query head of
    that (batch, kv head), on both decode kernels; the other kv head's heads,
    in the same call, stay within the bound of the oracle."""
    w = synth.WORKLOADS["tiny_mixkvq"].scaled(batch=1, n_kv_heads=2, n_q_heads=8, n_pages=1, n_resid=0,
                                              n_append=0, seed=1331)
    p = built(w)
    rec = p.gpu_record(0, 0)
    k = p.k_pre[:, :, :128].clone()
    v = p.v_pre[:, :, :128].clone()
    if part == "key":
        k[0, 0, 10, int(rec[100])] = 4.0e5     # a UINT2 channel: infinite scale
    else:
        v[0, 0, 9, 40] = -3.0e5                # a value group: infinite offset
    f = _flush_one(p, k, v)
    assert f & kvq.KVQ_FLAG_RANGE, f
    g = w.group
    for generic in (False, True):
        p.decode(n_pages=1, n_resid=0, generic=generic)
        torch.cuda.synchronize()
        out = p.out.cpu().numpy()
        for hq in range(g):
            assert not np.all(np.isfinite(out[0, hq])), (part, generic, hq)
        rec1 = p.gpu_record(0, 1)
        ref, _ = p.oracle_decode(0, 1, [p.oracle_page(0, 1, 0, rec1)], rec1, n_resid=0)
        assert np.all(np.isfinite(out[0, g:])) and np.all(rel_err(out[0, g:], ref) <= TOL), (part, generic)
