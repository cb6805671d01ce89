"""Pins of storage accounting, the residual state machine and the page layout.

* KIVI blog section 7: 419 840 bytes (410 KiB) for T=4096, D=128, G=32,
  r_K=0, r_V=128, b=2, e=f=2; 2 + 32/32 = 3 bits per quantized element;
* PN-Mix notes: 32 516 bytes (FP16 floats) and 52 740 bytes (float32) for the
  local component run, about 2.26 K bits at 32K quantized tokens;
* KIVI blog section 5: the fixed flash order's residual lengths at R=4, G=2;
* page layouts: pack/unpack round trips of every codec, 256-byte strides,
  MixKVQ / PN-Mix / QJL page sizes of the workloads.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import cache, flush, layout, storage
from oracle.quant import quantize_groups

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_kivi_storage_pin():
    g = gold("storage_pins.json")["kivi_form"]
    total = storage.kivi_bytes(g["T"], g["D"], g["G"], g["r_k"], g["r_v"], g["b"], g["e"], g["f"])
    assert total == g["total_kib"] * 1024
    assert 2 * g["T"] * g["D"] * g["f"] == g["unquantized_bytes"]
    assert (g["r_k"] + g["r_v"]) * g["D"] * g["f"] == g["residual_bytes"]
    assert storage.kivi_bits_per_element(g["b"], g["e"], g["G"]) == g["bits_per_quantized_element"]


def test_pnmix_storage_pins():
    g = gold("storage_pins.json")
    c = g["pnmix_component"]
    b16 = storage.pnmix_breakdown(h_kv_d=c["h_kv_d"], n_sink=c["n_sink"], n_quant=c["n_quant"],
                                  n_resid=c["n_resid"], float_bytes=2)
    b32 = storage.pnmix_breakdown(h_kv_d=c["h_kv_d"], n_sink=c["n_sink"], n_quant=c["n_quant"],
                                  n_resid=c["n_resid"], float_bytes=4)
    assert b16["total"] == c["bytes_fp16"]
    assert b32["total"] == c["bytes_fp32"]
    p = g["pnmix_32k"]
    bits = storage.pnmix_key_bits(d=p["d"], n_quant=p["n_quant"], n_sink=p["n_sink"])
    assert round(float(bits), 2) == p["approx_bits"]
    assert bits == Fraction(32768 * 9 // 4 + 32 * 16, 32800)


def test_kivi_residual_trace():
    g = gold("kivi_residual_trace.json")
    rows = cache.kivi_flash_trace(g["R"], g["G"], 9)
    for step, expect in g["table_rows"].items():
        assert list(rows[int(step) - 1][:4]) == expect
    assert [r.k_persist_full for r in rows] == g["persisted_k_lengths_9_steps"]
    assert [r.v_persist_full for r in rows] == g["persisted_v_lengths_9_steps"]
    kc, vc = rows[8].k_split, rows[8].v_split
    assert [len(kc[0]), len(kc[1])] == g["step9_key_split"]
    assert [len(vc[0]), len(vc[1])] == g["step9_value_split"]
    # mean persisted Key residual over full cycles is (R-1)/2
    R = 128
    trace = cache.kivi_flash_trace(R, 32, 4 * R)
    lens = [r.k_persist_full for r in trace]
    assert Fraction(sum(lens), len(lens)) == Fraction(R - 1, 2)
    # every step reads every token once, the Key history in whole segments of
    # R and the Value window as the newest tokens
    for t, r in enumerate(trace, start=1):
        for q_ids, f_ids in (r.k_split, r.v_split):
            assert list(q_ids) + list(f_ids) == list(range(1, t + 1))
        assert len(r.k_split[0]) % R == 0 and 1 <= r.k_compute_full <= R
        assert r.v_compute_full == min(t, R + 1)
    with pytest.raises(ValueError):
        cache.kivi_flash_trace(6, 4, 3)


def rand_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_mixkvq_page_roundtrip():
    rng = np.random.default_rng(0)
    for n16, n4 in ((16, 32), (1, 12), (0, 0), (3, 5), (128, 0), (0, 128)):
        perm = rng.permutation(128).astype(np.uint8)
        K = rand_bits(rng, (128, 128))
        V = rand_bits(rng, (128, 128))
        page = flush.flush_mixkvq_page(K, V, perm, n16, n4)
        geo = layout.mixkvq_geometry(n16, n4)
        assert page.size == geo["stride"] and geo["stride"] % 256 == 0
        u = layout.unpack_mixkvq_page(page, n16, n4, perm)
        n2 = 128 - n16 - n4
        assert np.array_equal(u["kbf"], K[:, perm[:n16].astype(int)].T)
        c4 = quantize_groups(K[:, perm[n16:n16 + n4].astype(int)].T, 4) if n4 else None
        if n4:
            for a, b in zip(u["k4"], c4):
                assert np.array_equal(a, b)
        if n2:
            c2 = quantize_groups(K[:, perm[n16 + n4:].astype(int)].T, 2)
            for a, b in zip(u["k2"], c2):
                assert np.array_equal(a, b)
        vq = flush.quantize_values(V)
        for a, b in zip(u["v"], vq):
            assert np.array_equal(a, b)
        assert not u["pad_codes"].any()
    assert layout.mixkvq_geometry(1, 12)["used"] == 256 + 18 * 256 + 18 * 32 + 6144


def test_pnmix_and_qjl_page_roundtrip():
    rng = np.random.default_rng(1)
    hi = np.zeros(128, bool)
    hi[rng.choice(128, 64, replace=False)] = True
    K = rand_bits(rng, (128, 128))
    V = rand_bits(rng, (128, 128))
    page = flush.flush_pnmix_page(K, V, hi)
    assert layout.pnmix_geometry(64)["used"] == 10752
    u = layout.unpack_pnmix_page(page, hi)
    assert u["codes"][hi].max() <= 7 and u["codes"][~hi].max() <= 1
    S = rand_bits(rng, (256, 128))
    pq = flush.flush_qjl_page(K, V, S)
    assert layout.qjl_geometry(256)["used"] == 10496
    uq = layout.unpack_qjl_page(pq, 256)
    from oracle.qjl import key_norms, sketch_bits
    assert np.array_equal(uq["bits"], sketch_bits(S, K))
    assert np.array_equal(uq["norms"], key_norms(K))


def test_one_bit_block_roundtrip():
    rng = np.random.default_rng(2)
    for n in (128, 256, 64):
        bits = rng.integers(0, 2, (n, 128)).astype(np.uint8)
        reg = layout.pack1_region(bits)
        assert np.array_equal(layout.unpack1_region(reg, n), bits)
    X = rng.integers(0, 4, (16, 8, 8)).astype(np.uint8)
    assert np.array_equal(layout.unpack2_block(layout.pack2_block(X)), X)
