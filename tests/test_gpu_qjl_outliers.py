"""GPU parity of the QJL outlier split (QJL page, outlier handling with
Figure 2: outlier channels fixed at the prompt, two independent sketch
instances) against the oracle.

* outlier records (kvq_select_channels on the prompt's Keys) bit-exact,
  also where column sums tie (integer-valued Keys);
* flushed pages (both instances' sign bits and norms, values) bit-exact;
* decode within 2e-3 of max |ref| per query head, for several (g, m, m_out),
  with and without residual tokens and with no pages;
* the fused decode + flush call: the same output bits as the decode call
  and the flushed page bit-exact.
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
BASE = synth.WORKLOADS["qjl_outlier_32k"]


def small(group=4, m=256, m_out=64, n_pages=3, n_resid=40, seed=0, n_out=8):
    return BASE.scaled(batch=2, n_kv_heads=2, n_q_heads=2 * group, n_pages=n_pages, n_resid=n_resid,
                       qjl_m=m, qjl_m_out=m_out, qjl_outliers=n_out, seed=BASE.seed + 600 + seed)


def built(w):
    print(f"\n[case] {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    return p


def check_records_and_pages(p):
    w = p.w
    assert int(p.flags[0].item()) == 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            rec = p.gpu_record(b, h)
            assert np.array_equal(rec, p.oracle_record(b, h)), (b, h)
            assert int(np.unpackbits(rec).sum()) == w.qjl_outliers
            for pg in range(w.n_pages):
                assert np.array_equal(p.gpu_page(b, h, pg), p.oracle_page(b, h, pg, rec)), (b, h, pg)


def check_decode(p, n_pages, n_resid, tag):
    out = p.out.cpu().numpy()
    g = p.g
    for b in range(p.w.batch):
        for h in range(p.w.n_kv_heads):
            rec = p.gpu_record(b, h)
            pages = [p.oracle_page(b, h, pg, rec) for pg in range(n_pages)]
            ref, _ = p.oracle_decode(b, h, pages, rec, n_resid=n_resid)
            err = rel_err(out[b, h * g:(h + 1) * g], ref)
            assert np.all(err <= TOL), (tag, b, h, err)


@pytest.mark.parametrize("group,m,m_out", [(4, 256, 64), (8, 256, 64), (8, 128, 128), (2, 192, 64)])
def test_split_select_flush_decode(group, m, m_out):
    w = small(group, m, m_out, seed=group)
    p = built(w)
    check_records_and_pages(p)
    p.decode()
    torch.cuda.synchronize()
    check_decode(p, w.n_pages, w.n_resid, f"g{group} m{m}+{m_out}")
    # no residual, then no pages (residual only)
    p.decode(n_resid=0)
    torch.cuda.synchronize()
    check_decode(p, w.n_pages, 0, "no residual")
    p.decode(n_pages=0)
    torch.cuda.synchronize()
    check_decode(p, 0, w.n_resid, "no pages")


def test_split_select_ties():
    """Integer-valued Keys on 0..3: many channels share the exact sum of |K|
    and the lower channel must win, as in the oracle."""
    w = small(n_pages=2, n_resid=0, seed=9, n_out=5)
    p = Pipeline(w)
    gen = torch.Generator(device="cpu").manual_seed(11)
    k = torch.randint(0, 4, tuple(p.k_pre.shape), generator=gen).to(torch.bfloat16)
    k[..., 7] = 3.0
    k[..., 90] = 3.0                                     # two channels tied at the top
    p.k_pre = k.cuda()
    p.select()
    p.flush_prefill()
    torch.cuda.synchronize()
    check_records_and_pages(p)
    p.decode()
    torch.cuda.synchronize()
    check_decode(p, w.n_pages, 0, "ties")


def test_split_fused_decode_flush():
    w = small(n_pages=3, n_resid=128, seed=21)
    p = built(w)
    p.decode()
    torch.cuda.synchronize()
    ref_out = p.out.clone()
    p.out.zero_()
    p.decode_flush()
    torch.cuda.synchronize()
    assert torch.equal(p.out, ref_out)
    assert int(p.flags[0].item()) == 0
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            rec = p.gpu_record(b, h)
            ref = p.oracle_flush(p.bits(p.resid_k[b, h]), p.bits(p.resid_v[b, h]), rec)
            assert np.array_equal(p.gpu_page(b, h, w.n_pages), ref), (b, h)
    check_decode(p, w.n_pages, 128, "fused")
