"""The C-ABI library loads, exports every entry point include/kvq.h declares,
and its host-only calls (geometry, storage accounting, argument validation)
agree with the oracle. No compute call is made here (no GPU needed)."""
import os
import re
import ctypes

import pytest

import mixed_precision_kv_amd as kvq
from oracle import layout, storage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:kvq_status|int32_t|const char\*)\s+(kvq_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvq.LIB_PATH):
        from mixed_precision_kv_amd.build import build
        build()
    return kvq.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(kvq.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert kvq.kvq_abi_version() == kvq.KVQ_ABI_VERSION == 4
    assert kvq.kvq_status_string(0) == "ok"


def test_config_struct_matches_header():
    assert ctypes.sizeof(kvq.KvqConfig) == 18 * 4 + 2 * 8 and kvq.KvqConfig.tau_bf16.offset == 72
    assert ctypes.sizeof(kvq.KvqStorage) == 9 * 8 + 8


@pytest.mark.parametrize("n16,n4", [(16, 32), (1, 12), (0, 0), (128, 0), (3, 7)])
def test_mixkvq_page_bytes(lib, n16, n4):
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 2, 8, 2, 10, n_bf16=n16, n_u4=n4)
    assert kvq.kvq_page_bytes(cfg) == layout.mixkvq_geometry(n16, n4)["stride"]
    assert kvq.kvq_mask_bytes(cfg) == 160


def test_pnmix_qjl_page_bytes(lib):
    cfg = kvq.make_config(kvq.KVQ_KEY_PNMIX, 1, 4, 1, 4, n_hi_pairs=32)
    assert kvq.kvq_page_bytes(cfg) == layout.pnmix_geometry(64)["stride"] == 10752
    assert kvq.kvq_mask_bytes(cfg) == 8
    cfg = kvq.make_config(kvq.KVQ_KEY_QJL, 1, 4, 1, 4, qjl_m=256)
    assert kvq.kvq_page_bytes(cfg) == layout.qjl_geometry(256)["stride"] == 10496
    assert kvq.kvq_mask_bytes(cfg) == 0


def test_qjl_outlier_split_config(lib):
    """QJL outlier split: page geometry and record size as the oracle packs
    them, storage by region, and the configurations it rejects."""
    cfg = kvq.make_config(kvq.KVQ_KEY_QJL, 2, 8, 2, 4, qjl_m=256, qjl_outliers=8, qjl_m_out=64)
    g = layout.qjl_geometry(256, 64)
    assert kvq.kvq_page_bytes(cfg) == g["stride"] and g["used"] == 16 * 320 + 512 + 6144
    assert kvq.kvq_mask_bytes(cfg) == 16
    st = kvq.kvq_storage_bytes(cfg, 1024, 0, 0)
    H, T = 4, 1024
    assert st["key_codes"] == H * T * 320 // 8 and st["key_meta"] == H * T * 4 and st["selection"] == H * 16
    assert abs(st["key_bits_per_element"] - (320 + 32) / 128) < 1e-12
    for kw, status in ((dict(qjl_outliers=8, qjl_m_out=0), kvq.KVQ_INVALID_ARG),
                       (dict(qjl_outliers=0, qjl_m_out=64), kvq.KVQ_INVALID_ARG),
                       (dict(qjl_outliers=65, qjl_m_out=64), kvq.KVQ_INVALID_ARG),
                       (dict(qjl_outliers=8, qjl_m_out=96), kvq.KVQ_INVALID_ARG),
                       (dict(qjl_outliers=8, qjl_m_out=192), kvq.KVQ_UNSUPPORTED)):
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_page_bytes(kvq.make_config(kvq.KVQ_KEY_QJL, 1, 4, 1, 4, qjl_m=256, **kw))
        assert e.value.status == status, kw
    # selection: plain QJL has none; the split needs K and a record buffer (rejected before launch)
    plain = kvq.make_config(kvq.KVQ_KEY_QJL, 1, 4, 1, 4, qjl_m=256)
    assert lib.kvq_select_channels(ctypes.byref(plain), None, 0, 0, None, 10, 10, None, None) == kvq.KVQ_UNSUPPORTED
    assert lib.kvq_select_channels(ctypes.byref(cfg), None, 0, 0, None, 10, 10, None, None) == kvq.KVQ_INVALID_ARG


def test_storage_matches_oracle(lib):
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 8, 32, 8, 64, n_bf16=1, n_u4=12)
    got = kvq.kvq_storage_bytes(cfg, 8192, 128, 0)
    ref = storage.mixkvq_breakdown(n_kv_heads=64, d=128, n16=1, n4=12, n_quant=8192, n_resid=128)
    assert got["key_full"] == ref["k_bf16"] and got["key_codes"] == ref["k_codes"]
    assert got["key_meta"] == ref["k_meta"] and got["value_codes"] == ref["v_codes"]
    assert got["value_meta"] == ref["v_meta"] and got["residual"] == ref["residual"]
    assert got["total"] == ref["total"]
    # per-flush reselection: one selection record per page
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 8, 32, 8, 64, n_bf16=1, n_u4=12, page_records=1)
    got = kvq.kvq_storage_bytes(cfg, 8192, 128, 0)
    ref = storage.mixkvq_breakdown(n_kv_heads=64, d=128, n16=1, n4=12, n_quant=8192, n_resid=128,
                                   per_page_records=True)
    assert got["selection"] == ref["mask"] == 64 * 64 * 160 and got["total"] == ref["total"]
    # PN-Mix at the 32K configuration: about 2.26 K bits (residual excluded)
    cfg = kvq.make_config(kvq.KVQ_KEY_PNMIX, 1, 1, 1, 256, n_hi_pairs=32)
    got = kvq.kvq_storage_bytes(cfg, 32768, 0, 32)
    assert abs(got["key_bits_per_element"] - float(storage.pnmix_key_bits(d=128, n_quant=32768, n_sink=32))) < 1e-12
    pn = storage.pnmix_breakdown(h_kv_d=128, n_sink=32, n_quant=32768, n_resid=128)
    got = kvq.kvq_storage_bytes(cfg, 32768, 128, 32)
    assert got["key_codes"] == pn["k_codes"] and got["key_meta"] == pn["k_meta"]
    assert got["sink"] == pn["sink"] and got["residual"] == pn["residual"] and got["selection"] == pn["mask"]


def test_validation_rejects_before_launch(lib):
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 1, 4, 1, 8, n_bf16=16, n_u4=32)
    bad = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 1, 4, 1, 8, head_dim=64)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_page_bytes(bad)
    assert e.value.status == kvq.KVQ_UNSUPPORTED
    for field, value, status in (("n_q_heads", 6, kvq.KVQ_UNSUPPORTED), ("n_kv_heads", 3, kvq.KVQ_INVALID_ARG),
                                 ("abi_version", 3, kvq.KVQ_INVALID_ARG), ("reserved", 1, kvq.KVQ_INVALID_ARG),
                                 ("select_mode", 2, kvq.KVQ_INVALID_ARG), ("decode_path", 2, kvq.KVQ_INVALID_ARG),
                                 ("qjl_outliers", 8, kvq.KVQ_INVALID_ARG),
                                 ("n_bf16", 120, kvq.KVQ_INVALID_ARG), ("key_mode", 7, kvq.KVQ_INVALID_ARG)):
        c = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 1, 4, 1, 8, n_bf16=16, n_u4=32)
        setattr(c, field, value)
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_page_bytes(c)
        assert e.value.status == status
    S = lib
    st = S.kvq_select_channels(ctypes.byref(cfg), None, 10, 10, None, 10, 10, None, None)
    assert st == kvq.KVQ_INVALID_ARG
    st = S.kvq_flush_quantize(ctypes.byref(cfg), 16, 16, 128, 1, 16, None, 16, None, 0, 8, 16, None)
    assert st == kvq.KVQ_CAPACITY
    st = S.kvq_flush_quantize(ctypes.byref(cfg), 8, 16, 128, 1, 16, None, 16, None, 0, 0, 16, None)
    assert st == kvq.KVQ_INVALID_ARG                               # misaligned source
    st = S.kvq_decode_attention(ctypes.byref(cfg), 16, 16, None, 0, 2, 16, None, None, None, 0, 16, 16, 129, 129,
                                0.088, 16, 16, 1 << 20, None)
    assert st == kvq.KVQ_INVALID_ARG                               # residual longer than 128
    st = S.kvq_decode_attention(ctypes.byref(cfg), 16, 16, None, 0, 2, 16, None, None, None, 0, None, None, 0, 0,
                                0.088, 16, 16, 16, None)
    assert st == kvq.KVQ_WORKSPACE_TOO_SMALL
    # the fused call fails as a whole when either half's check fails
    big = 1 << 30
    st = S.kvq_decode_attention_flush(ctypes.byref(cfg), 16, 16, None, 0, 2, 16, None, None, None, 0, None, None, 0, 0,
                                      0.088, 16, 16, big, 16, 16, 128, 1, 8, 16, None)
    assert st == kvq.KVQ_CAPACITY                                  # flush past max_pages
    st = S.kvq_decode_attention_flush(ctypes.byref(cfg), 16, 16, None, 0, 2, 16, None, None, None, 0, None, None, 0, 0,
                                      0.088, 16, 16, big, 16, 16, 128, 1, 2, None, None)
    assert st == kvq.KVQ_INVALID_ARG                               # no status word
    st = S.kvq_decode_attention_flush(ctypes.byref(cfg), 16, 16, None, 0, 2, 16, None, None, None, 0, 16, 16, 129, 129,
                                      0.088, 16, 16, big, 16, 16, 128, 1, 2, 16, None)
    assert st == kvq.KVQ_INVALID_ARG                               # decode half: residual longer than 128
    st = S.kvq_decode_attention_flush(ctypes.byref(cfg), 16, 16, None, 0, 2, 16, None, None, None, 0, None, None, 0, 0,
                                      0.088, 16, 16, 16, 16, 16, 128, 1, 2, 16, None)
    assert st == kvq.KVQ_WORKSPACE_TOO_SMALL
    # page tables: the logical range is checked against table_stride, the
    # table's alignment and stride are checked
    st = S.kvq_flush_quantize(ctypes.byref(cfg), 16, 16, 128, 1, 16, None, 16, 16, 4, 4, 16, None)
    assert st == kvq.KVQ_CAPACITY                                  # first_page + n_pages > table_stride
    st = S.kvq_flush_quantize(ctypes.byref(cfg), 16, 16, 128, 1, 16, None, 16, 18, 8, 0, 16, None)
    assert st == kvq.KVQ_INVALID_ARG                               # misaligned table
    st = S.kvq_decode_attention(ctypes.byref(cfg), 16, 16, 16, 4, 5, 16, None, None, None, 0, None, None, 0, 0,
                                0.088, 16, 16, big, None)
    assert st == kvq.KVQ_INVALID_ARG                               # n_pages > table_stride
    st = S.kvq_decode_attention(ctypes.byref(cfg), 16, 16, 16, 0, 1, 16, None, None, None, 0, None, None, 0, 0,
                                0.088, 16, 16, big, None)
    assert st == kvq.KVQ_INVALID_ARG                               # table_stride 0
    qcfg = kvq.make_config(kvq.KVQ_KEY_QJL, 1, 4, 1, 8, qjl_m=256)
    st = S.kvq_select_channels(ctypes.byref(qcfg), 16, 10, 10, 16, 10, 10, 16, None)
    assert st == kvq.KVQ_UNSUPPORTED
    assert kvq.kvq_workspace_bytes(cfg, 8) > 0
    # the read-stream reference checks its buffers before it launches
    assert S.kvq_read_stream(16, 0, 16, 0, None) == kvq.KVQ_OK                      # nothing to read
    assert S.kvq_read_stream(8, 64, 16, 4, None) == kvq.KVQ_INVALID_ARG             # misaligned source
    assert S.kvq_read_stream(16, 40, 16, 4, None) == kvq.KVQ_INVALID_ARG            # not whole 16-byte loads
    assert S.kvq_read_stream(16, 16384 + 16, 16, 4, None) == kvq.KVQ_WORKSPACE_TOO_SMALL   # 2 chunks, 1 word


def test_fifo_validation_rejects_before_launch(lib):
    """The KIVI Value FIFO's entry points check their arguments before any
    launch (every call here fails a check, so no pointer is touched)."""
    S = lib
    cfg = kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 1, 4, 1, 8, n_bf16=16, n_u4=32)
    rec = kvq.with_fields(cfg, page_records=1)
    big = 1 << 30
    # Key seal: the flush's checks, and no per-page records
    assert S.kvq_flush_keys(ctypes.byref(cfg), 16, 16, 128, 1, 16, None, 16, None, 0, 8, 16, None) == kvq.KVQ_CAPACITY
    assert S.kvq_flush_keys(ctypes.byref(cfg), 8, 8, 128, 1, 16, None, 16, None, 0, 0, 16, None) == kvq.KVQ_INVALID_ARG
    assert S.kvq_flush_keys(ctypes.byref(rec), 16, 16, 128, 1, 16, None, 16, None, 0, 0, 16, None) == kvq.KVQ_UNSUPPORTED
    # Value push
    push = S.kvq_value_push
    assert push(ctypes.byref(cfg), 16, 128, 0, 0, 16, 16, None, 0, 16, None) == kvq.KVQ_OK            # nothing to push
    assert push(ctypes.byref(cfg), 16, 128, -1, 0, 16, 16, None, 0, 16, None) == kvq.KVQ_INVALID_ARG
    assert push(ctypes.byref(cfg), 16, 4, 8, 0, 16, 16, None, 0, 16, None) == kvq.KVQ_INVALID_ARG     # stride < rows
    assert push(ctypes.byref(cfg), 8, 128, 1, 0, 16, 16, None, 0, 16, None) == kvq.KVQ_INVALID_ARG    # misaligned rows
    assert push(ctypes.byref(cfg), 16, 128, 1, 0, 16, 16, None, 0, None, None) == kvq.KVQ_INVALID_ARG  # no status word
    assert push(ctypes.byref(cfg), 16, 2048, 1, 8 * 128, 16, 16, None, 0, 16, None) == kvq.KVQ_CAPACITY   # page 8
    assert push(ctypes.byref(cfg), 16, 2048, 1, 4 * 128, 16, 16, 16, 4, 16, None) == kvq.KVQ_CAPACITY   # past the table
    assert push(ctypes.byref(rec), 16, 128, 1, 0, 16, 16, None, 0, 16, None) == kvq.KVQ_UNSUPPORTED

    # FIFO decode: cfg, q, arena, table, table_stride, n_pages, n_vq, mask, qjl_s, resid_k, n_kres, kres_stride,
    # vwin, n_vwin, vwin_stride, scale, out, workspace, workspace_bytes, stream
    def fifo(c, n_pages, n_vq, n_kres, n_vwin, vwin=16, ws_bytes=big):
        return S.kvq_decode_attention_fifo(ctypes.byref(c), 16, 16, None, 0, n_pages, n_vq, 16, None, 16, n_kres,
                                           max(n_kres, 1), vwin, n_vwin, max(n_vwin, 1), 0.088, 16, 16, ws_bytes, None)
    assert fifo(cfg, 2, 100, 129, 285) == kvq.KVQ_INVALID_ARG          # Key residual longer than 128
    assert fifo(cfg, 2, 0, 1, 257) == kvq.KVQ_INVALID_ARG              # window longer than 256
    assert fifo(cfg, 1, 129, 1, 0) == kvq.KVQ_INVALID_ARG              # quantized Values past the pages
    assert fifo(cfg, 1, 100, 0, -1) == kvq.KVQ_INVALID_ARG             # negative window
    assert fifo(cfg, 2, 100, 10, 100) == kvq.KVQ_INVALID_ARG           # n_pages 128 + n_kres != n_vq + n_vwin
    assert fifo(cfg, 2, 100, 10, 166, vwin=8) == kvq.KVQ_INVALID_ARG   # misaligned window
    assert fifo(cfg, 2, 100, 10, 166, vwin=None) == kvq.KVQ_INVALID_ARG
    assert fifo(cfg, 2, 100, 10, 166, ws_bytes=16) == kvq.KVQ_WORKSPACE_TOO_SMALL
    assert fifo(rec, 2, 100, 10, 166) == kvq.KVQ_UNSUPPORTED


def test_threshold_config(lib):
    """Threshold tiers: the thresholds' domain is checked; the page stride is
    the largest page any counts within the capacities need (fewer BF16
    channels can mean a larger code region)."""
    def cfg(**kw):
        return kvq.make_config(kvq.KVQ_KEY_MIXKVQ, 1, 4, 1, 8, n_bf16=1, n_u4=12,
                               select_mode=kvq.KVQ_SELECT_THRESHOLD, **kw)
    c = cfg(tau_bf16=1.44, tau_u4=0.79)
    want = max(layout.mixkvq_geometry(a, b)["stride"] for a in range(2) for b in range(13))
    assert kvq.kvq_page_bytes(c) == want >= layout.mixkvq_geometry(1, 12)["stride"]
    for t16, t4 in ((float("nan"), 0.5), (1.0, float("inf")), (1e-300, 0.5), (1.0, 2.0 ** 950)):
        with pytest.raises(kvq.KvqError) as e:
            kvq.kvq_page_bytes(cfg(tau_bf16=t16, tau_u4=t4))
        assert e.value.status == kvq.KVQ_INVALID_ARG
    kvq.kvq_page_bytes(cfg(tau_bf16=0.0, tau_u4=-1.5))   # zero and negative thresholds are valid
    with pytest.raises(kvq.KvqError) as e:               # threshold tiers are MixKVQ's
        kvq.kvq_page_bytes(kvq.make_config(kvq.KVQ_KEY_PNMIX, 1, 4, 1, 8, select_mode=kvq.KVQ_SELECT_THRESHOLD))
    assert e.value.status == kvq.KVQ_INVALID_ARG
    with pytest.raises(kvq.KvqError) as e:               # no mean |Q| from the running accumulator
        kvq.kvq_page_bytes(cfg(tau_bf16=1.0, tau_u4=0.5, page_records=1))
    assert e.value.status == kvq.KVQ_UNSUPPORTED
