"""GPU parity of libkvq against the oracle (select, flush, decode).

Selection records and packed pages must be bit-exact; decode outputs must be
within max_d |o - o_ref| <= 2e-3 * max_d |o_ref| per query head, where o_ref is
the oracle's float64 attention over the same dequantized cache. Small
workloads are checked on every (batch, kv head) and every page; they span
several tiles, several splits and a ragged residual.
"""
import numpy as np
import pytest
import torch

import kvq_synth as synth
from kvq_harness import Pipeline, rel_err

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a ROCm GPU")]

TOL = 2e-3


def small(name, **kw):
    return synth.WORKLOADS[name].scaled(**kw)


CASES = {
    "tiny_mixkvq": synth.WORKLOADS["tiny_mixkvq"],
    "mixkvq_small_g4": small("llama8b_8k", batch=2, n_kv_heads=2, n_q_heads=8, n_pages=5, n_resid=77, seed=11),
    "mixkvq_small_g8": small("qwen32b_32k", batch=1, n_kv_heads=2, n_q_heads=16, n_pages=6, n_resid=0, seed=12),
    "mixkvq_g2_tiers": small("tiny_mixkvq", batch=2, n_kv_heads=1, n_q_heads=2, n_pages=3, n_resid=128,
                             n_bf16=3, n_u4=5, seed=13),
    "mixkvq_g1_allbf16": small("tiny_mixkvq", batch=1, n_kv_heads=2, n_q_heads=2, n_pages=2, n_resid=5,
                               n_bf16=128, n_u4=0, seed=14),
    "pnmix_small": small("pnmix_16k", batch=2, n_kv_heads=2, n_q_heads=8, n_pages=3, n_resid=50, seed=15),
    "qjl_small": small("qjl_32k", batch=2, n_kv_heads=2, n_q_heads=8, n_pages=3, n_resid=20, seed=16),
    "qjl_g8": small("qjl_32k", batch=1, n_kv_heads=1, n_q_heads=8, n_pages=4, n_resid=0, seed=17),
}


@pytest.fixture(scope="module", params=sorted(CASES))
def run(request):
    w = CASES[request.param]
    print(f"\n[case] {request.param}: {w}", flush=True)
    p = Pipeline(w)
    p.select()
    p.flush_prefill()
    p.decode()
    torch.cuda.synchronize()
    return request.param, p


def test_select_bit_exact(run):
    name, p = run
    if p.w.key_mode == synth.QJL:
        pytest.skip("QJL has no selection")
    for b in range(p.w.batch):
        for h in range(p.w.n_kv_heads):
            assert np.array_equal(p.gpu_record(b, h), p.oracle_record(b, h)), (name, b, h)


def test_flush_bit_exact(run):
    name, p = run
    assert int(p.flags[0].item()) == 0
    for b in range(p.w.batch):
        for h in range(p.w.n_kv_heads):
            rec = p.gpu_record(b, h) if p.w.key_mode != synth.QJL else None
            for pg in range(p.w.n_pages):
                ref = p.oracle_page(b, h, pg, rec)
                got = p.gpu_page(b, h, pg)
                if not np.array_equal(got, ref):
                    bad = np.nonzero(got != ref)[0]
                    raise AssertionError(f"{name} b{b} h{h} page{pg}: {bad.size} bytes differ, first at {bad[:8]}")


def test_decode_within_tolerance(run):
    name, p = run
    out = p.out.cpu().numpy()
    g = p.g
    worst = 0.0
    for b in range(p.w.batch):
        for h in range(p.w.n_kv_heads):
            rec = p.gpu_record(b, h) if p.w.key_mode != synth.QJL else None
            pages = [p.oracle_page(b, h, pg, rec) for pg in range(p.w.n_pages)]
            ref, _ = p.oracle_decode(b, h, pages, rec)
            err = rel_err(out[b, h * g:(h + 1) * g], ref)
            worst = max(worst, float(err.max()))
            assert np.all(err <= TOL), (name, b, h, err)
    print(f"[decode] {name}: worst relative error {worst:.3e}")
