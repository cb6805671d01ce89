"""Python binding of libkvq (the C ABI in include/kvq.h).

Argument marshalling only: every step of the hot path runs in the HIP
kernels of libkvq.so. Tensors are PyTorch-ROCm tensors (used for device
memory and streams); the functions keep the C names. There is no CPU
fallback: importing works without a GPU, but any call that needs the library
raises if libkvq.so is missing, and device calls need a ROCm device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

KVQ_ABI_VERSION = 4
KVQ_OK, KVQ_INVALID_ARG, KVQ_UNSUPPORTED, KVQ_WORKSPACE_TOO_SMALL, KVQ_CAPACITY, KVQ_HIP_ERROR = range(6)
KVQ_KEY_MIXKVQ, KVQ_KEY_PNMIX, KVQ_KEY_QJL = 0, 1, 2
KVQ_PAIR_HALF_SPLIT, KVQ_PAIR_ADJACENT = 0, 1
KVQ_SELECT_COUNT, KVQ_SELECT_THRESHOLD = 0, 1
KVQ_DECODE_AUTO, KVQ_DECODE_GENERIC = 0, 1
KVQ_FLAG_NONFINITE, KVQ_FLAG_SPAN, KVQ_FLAG_MASK, KVQ_FLAG_RANGE, KVQ_FLAG_TABLE = 1, 2, 4, 8, 16

EXPORTED = (
    "kvq_abi_version", "kvq_status_string", "kvq_page_bytes", "kvq_mask_bytes",
    "kvq_workspace_bytes", "kvq_storage_bytes", "kvq_select_channels",
    "kvq_flush_quantize", "kvq_decode_attention", "kvq_decode_attention_flush",
    "kvq_accumulate_query", "kvq_flush_reselect", "kvq_decode_attention_noalloc",
    "kvq_flush_keys", "kvq_value_push", "kvq_decode_attention_fifo", "kvq_read_stream",
)
KVQ_NOALLOC_SCRATCH_BYTES = 16 << 20


class KvqConfig(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("key_mode", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("max_pages", ctypes.c_int32), ("n_bf16", ctypes.c_int32), ("n_u4", ctypes.c_int32),
        ("pair_layout", ctypes.c_int32), ("n_hi_pairs", ctypes.c_int32), ("qjl_m", ctypes.c_int32),
        ("page_records", ctypes.c_int32), ("qjl_outliers", ctypes.c_int32),
        ("qjl_m_out", ctypes.c_int32), ("select_mode", ctypes.c_int32), ("decode_path", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("tau_bf16", ctypes.c_double), ("tau_u4", ctypes.c_double),
    ]


class KvqStorage(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "key_full", "key_codes", "key_meta", "value_codes", "value_meta", "residual", "sink",
        "selection", "total")] + [("key_bits_per_element", ctypes.c_double)]


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {kvq_status_string(status)} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libkvq.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libkvq is not built ({path} missing); run `python -m mixed_precision_kv_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(KvqConfig)
    sig = {
        "kvq_abi_version": (I32, []),
        "kvq_status_string": (ctypes.c_char_p, [I32]),
        "kvq_page_bytes": (I32, [cfgp, ctypes.POINTER(SZ)]),
        "kvq_mask_bytes": (I32, [cfgp, ctypes.POINTER(SZ)]),
        "kvq_workspace_bytes": (I32, [cfgp, I32, ctypes.POINTER(SZ)]),
        "kvq_storage_bytes": (I32, [cfgp, I64, I32, I32, ctypes.POINTER(KvqStorage)]),
        "kvq_select_channels": (I32, [cfgp, P, I64, I64, P, I64, I64, P, P]),
        "kvq_flush_quantize": (I32, [cfgp, P, P, I64, I32, P, P, P, P, I32, I32, P, P]),
        "kvq_decode_attention": (I32, [cfgp, P, P, P, I32, I32, P, P, P, P, I32, P, P, I32, I32, ctypes.c_float,
                                       P, P, SZ, P]),
        "kvq_decode_attention_flush": (I32, [cfgp, P, P, P, I32, I32, P, P, P, P, I32, P, P, I32, I32,
                                             ctypes.c_float, P, P, SZ, P, P, I64, I32, I32, P, P]),
        "kvq_decode_attention_noalloc": (I32, [cfgp, P, P, P, I32, I32, P, P, P, P, I32, P, P, I32, I32,
                                               ctypes.c_float, P, P]),
        "kvq_flush_keys": (I32, [cfgp, P, P, I64, I32, P, P, P, P, I32, I32, P, P]),
        "kvq_value_push": (I32, [cfgp, P, I64, I32, I32, P, P, P, I32, P, P]),
        "kvq_decode_attention_fifo": (I32, [cfgp, P, P, P, I32, I32, I32, P, P, P, I32, I32, P, I32, I32,
                                            ctypes.c_float, P, P, SZ, P]),
        "kvq_accumulate_query": (I32, [cfgp, P, I64, I64, P, P]),
        "kvq_flush_reselect": (I32, [cfgp, P, P, I64, I32, P, P, P, P, I32, I32, P, P]),
        "kvq_read_stream": (I32, [P, SZ, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def make_config(key_mode: int, batch: int, n_q_heads: int, n_kv_heads: int, max_pages: int, *,
                n_bf16: int = 0, n_u4: int = 0, pair_layout: int = KVQ_PAIR_HALF_SPLIT,
                n_hi_pairs: int = 32, qjl_m: int = 256, head_dim: int = 128, page_records: int = 0,
                qjl_outliers: int = 0, qjl_m_out: int = 0, select_mode: int = KVQ_SELECT_COUNT,
                tau_bf16: float = 0.0, tau_u4: float = 0.0, decode_path: int = KVQ_DECODE_AUTO) -> KvqConfig:
    c = KvqConfig()
    c.abi_version = KVQ_ABI_VERSION
    c.key_mode = key_mode
    c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim = batch, n_q_heads, n_kv_heads, head_dim
    c.max_pages = max_pages
    c.n_bf16, c.n_u4 = n_bf16, n_u4
    c.pair_layout, c.n_hi_pairs, c.qjl_m = pair_layout, n_hi_pairs, qjl_m
    c.page_records = page_records
    c.qjl_outliers, c.qjl_m_out = qjl_outliers, qjl_m_out
    c.select_mode, c.tau_bf16, c.tau_u4 = select_mode, tau_bf16, tau_u4
    c.decode_path = decode_path
    return c


def with_fields(cfg: KvqConfig, **kw) -> KvqConfig:
    """A copy of cfg with some fields replaced (e.g. decode_path)."""
    c = KvqConfig()
    ctypes.pointer(c)[0] = cfg
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _ptr(x) -> Optional[int]:
    """Device (or host) address of a tensor; the C ABI takes dense buffers only."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("libkvq needs contiguous tensors (pass .contiguous())")
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != KVQ_OK:
        raise KvqError(fn, status)


def kvq_abi_version() -> int:
    return load().kvq_abi_version()


def kvq_status_string(status: int) -> str:
    return load().kvq_status_string(status).decode()


def kvq_page_bytes(cfg: KvqConfig) -> int:
    out = ctypes.c_size_t()
    _check("kvq_page_bytes", load().kvq_page_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def kvq_mask_bytes(cfg: KvqConfig) -> int:
    out = ctypes.c_size_t()
    _check("kvq_mask_bytes", load().kvq_mask_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def kvq_workspace_bytes(cfg: KvqConfig, n_pages: int) -> int:
    out = ctypes.c_size_t()
    _check("kvq_workspace_bytes", load().kvq_workspace_bytes(ctypes.byref(cfg), n_pages, ctypes.byref(out)))
    return out.value


def kvq_storage_bytes(cfg: KvqConfig, n_quant_tokens: int, n_resid: int, n_sink: int) -> dict:
    out = KvqStorage()
    _check("kvq_storage_bytes",
           load().kvq_storage_bytes(ctypes.byref(cfg), n_quant_tokens, n_resid, n_sink, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in KvqStorage._fields_}


def kvq_select_channels(cfg, q_pre, l_q, k_pre, l_k, mask_out, *, q_stride=None, k_stride=None, stream=None):
    """q_pre [B,Hq,q_stride,128], k_pre [B,Hkv,k_stride,128] bf16 (device pointers or tensors);
    the QJL outlier selection reads no queries (q_pre None, l_q 0)."""
    q_stride = l_q if q_stride is None else q_stride
    k_stride = l_k if k_stride is None else k_stride
    _check("kvq_select_channels", load().kvq_select_channels(
        ctypes.byref(cfg), _ptr(q_pre), l_q, q_stride, _ptr(k_pre), l_k, k_stride, _ptr(mask_out),
        _stream(stream)))


def kvq_flush_quantize(cfg, k_src, v_src, src_stride, n_pages, mask, qjl_s, page_arena, first_page,
                       status_flags, *, page_table=None, table_stride=0, stream=None):
    _check("kvq_flush_quantize", load().kvq_flush_quantize(
        ctypes.byref(cfg), _ptr(k_src), _ptr(v_src), src_stride, n_pages, _ptr(mask), _ptr(qjl_s),
        _ptr(page_arena), _ptr(page_table), table_stride, first_page, _ptr(status_flags), _stream(stream)))


def kvq_accumulate_query(cfg, q, l_q, q_stride, q_accum, *, stream=None):
    _check("kvq_accumulate_query", load().kvq_accumulate_query(
        ctypes.byref(cfg), _ptr(q), l_q, q_stride, _ptr(q_accum), _stream(stream)))


def kvq_flush_reselect(cfg, k_src, v_src, src_stride, n_pages, q_accum, page_records, page_arena, first_page,
                       status_flags, *, page_table=None, table_stride=0, stream=None):
    _check("kvq_flush_reselect", load().kvq_flush_reselect(
        ctypes.byref(cfg), _ptr(k_src), _ptr(v_src), src_stride, n_pages, _ptr(q_accum), _ptr(page_records),
        _ptr(page_arena), _ptr(page_table), table_stride, first_page, _ptr(status_flags), _stream(stream)))


def kvq_decode_attention_flush(cfg, q, page_arena, n_pages, mask, qjl_s, sink_k, sink_v, n_sink, resid_k,
                               resid_v, n_resid, resid_stride, softmax_scale, out, workspace, workspace_bytes,
                               flush_k_src, flush_v_src, flush_src_stride, n_flush_pages, flush_first_page,
                               status_flags, *, page_table=None, table_stride=0, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("kvq_decode_attention_flush", load().kvq_decode_attention_flush(
        ctypes.byref(cfg), _ptr(q), _ptr(page_arena), _ptr(page_table), table_stride, n_pages, _ptr(mask),
        _ptr(qjl_s), _ptr(sink_k),
        _ptr(sink_v), n_sink, _ptr(resid_k), _ptr(resid_v), n_resid, resid_stride, softmax_scale, _ptr(out),
        _ptr(workspace), workspace_bytes, _ptr(flush_k_src), _ptr(flush_v_src), flush_src_stride, n_flush_pages,
        flush_first_page, _ptr(status_flags), _stream(stream)))


def kvq_decode_attention(cfg, q, page_arena, n_pages, mask, qjl_s, sink_k, sink_v, n_sink, resid_k, resid_v,
                         n_resid, resid_stride, softmax_scale, out, workspace, workspace_bytes=None, *,
                         page_table=None, table_stride=0, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("kvq_decode_attention", load().kvq_decode_attention(
        ctypes.byref(cfg), _ptr(q), _ptr(page_arena), _ptr(page_table), table_stride, n_pages, _ptr(mask),
        _ptr(qjl_s), _ptr(sink_k),
        _ptr(sink_v), n_sink, _ptr(resid_k), _ptr(resid_v), n_resid, resid_stride, softmax_scale, _ptr(out),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def kvq_decode_attention_noalloc(cfg, q, page_arena, n_pages, mask, qjl_s, sink_k, sink_v, n_sink, resid_k, resid_v,
                                 n_resid, resid_stride, softmax_scale, out, *, page_table=None, table_stride=0,
                                 stream=None):
    """kvq_decode_attention with the library's per-GPU scratch instead of a workspace."""
    _check("kvq_decode_attention_noalloc", load().kvq_decode_attention_noalloc(
        ctypes.byref(cfg), _ptr(q), _ptr(page_arena), _ptr(page_table), table_stride, n_pages, _ptr(mask),
        _ptr(qjl_s), _ptr(sink_k), _ptr(sink_v), n_sink, _ptr(resid_k), _ptr(resid_v), n_resid, resid_stride,
        softmax_scale, _ptr(out), _stream(stream)))


def kvq_read_stream(src, nbytes, sink, sink_bytes, *, stream=None):
    """The measurement read-stream reference: one XOR word per 16 KB of src."""
    _check("kvq_read_stream", load().kvq_read_stream(_ptr(src), nbytes, _ptr(sink), sink_bytes, _stream(stream)))


def kvq_flush_keys(cfg, k_src, v_src, src_stride, n_pages, mask, qjl_s, page_arena, first_page, status_flags, *,
                   page_table=None, table_stride=0, stream=None):
    """The Value-FIFO seal: Keys packed, the pages' Value parts cleared."""
    _check("kvq_flush_keys", load().kvq_flush_keys(
        ctypes.byref(cfg), _ptr(k_src), _ptr(v_src), src_stride, n_pages, _ptr(mask), _ptr(qjl_s),
        _ptr(page_arena), _ptr(page_table), table_stride, first_page, _ptr(status_flags), _stream(stream)))


def kvq_value_push(cfg, v_src, src_stride, n_rows, first_token, mask, page_arena, status_flags, *,
                   page_table=None, table_stride=0, stream=None):
    _check("kvq_value_push", load().kvq_value_push(
        ctypes.byref(cfg), _ptr(v_src), src_stride, n_rows, first_token, _ptr(mask), _ptr(page_arena),
        _ptr(page_table), table_stride, _ptr(status_flags), _stream(stream)))


def kvq_decode_attention_fifo(cfg, q, page_arena, n_pages, n_vq, mask, qjl_s, resid_k, n_kres, kres_stride, vwin,
                              n_vwin, vwin_stride, softmax_scale, out, workspace, workspace_bytes=None, *,
                              page_table=None, table_stride=0, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("kvq_decode_attention_fifo", load().kvq_decode_attention_fifo(
        ctypes.byref(cfg), _ptr(q), _ptr(page_arena), _ptr(page_table), table_stride, n_pages, n_vq, _ptr(mask),
        _ptr(qjl_s), _ptr(resid_k), n_kres, kres_stride, _ptr(vwin), n_vwin, vwin_stride, softmax_scale, _ptr(out),
        _ptr(workspace), workspace_bytes, _stream(stream)))
