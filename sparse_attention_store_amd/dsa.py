"""Thin ctypes binding of libdsa (include/dsa.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU (torch provides device
memory and the current stream), passes raw pointers and sizes to the C ABI, and raises
DsaError on a non-zero status.  No arithmetic of the method happens here, and there is
no fallback: if the HIP library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

PAGE_SIZE = 64
INDEX_PAGE_BYTES = 8448
INDEX_MXFP4_PAGE_BYTES = 4352
LATENT_PAGE_BYTES = 41984
TOPK_MAX = 2048
PROBE_SINK_WORDS = 2048

_STATUS = {0: "DSA_OK", 1: "DSA_ERR_ARG", 2: "DSA_ERR_UNSUPPORTED", 3: "DSA_ERR_WORKSPACE",
           4: "DSA_ERR_HIP", 5: "DSA_ERR_DEVICE_CHECK"}


class DsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class _Pages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("pt_stride", ctypes.c_int64),
                ("num_reqs", ctypes.c_int32), ("num_pages", ctypes.c_int64)]


class _Rows(ctypes.Structure):
    _fields_ = [("req", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("n", ctypes.c_int32),
                ("group", ctypes.c_int32), ("max_pos", ctypes.c_int32)]


class _Rule(ctypes.Structure):
    _fields_ = [("indexer_types", ctypes.c_char_p), ("n_types", ctypes.c_int32),
                ("cli_factor", ctypes.c_int32), ("topk_pattern", ctypes.c_char_p),
                ("n_pattern", ctypes.c_int32), ("topk_freq", ctypes.c_int32),
                ("skip_topk_offset", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdsa.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    P, R = ctypes.POINTER(_Pages), ctypes.POINTER(_Rows)
    sigs = {
        "dsa_abi_version": ([], ctypes.c_int),
        "dsa_last_error": ([], ctypes.c_char_p),
        "dsa_layer_is_shared": ([ctypes.POINTER(_Rule), i32], ctypes.c_int),
        "dsa_mtp_seed_width": ([i32, i32], i32),
        "dsa_mtp_carry_allowed": ([i32], ctypes.c_int),
        "dsa_quant_fp8": ([p, i64, p, p, p], ctypes.c_int),
        "dsa_index_k_store": ([p, R, P, p, f64, f64, p], ctypes.c_int),
        "dsa_index_k_store_mxfp4": ([p, R, P, p, f64, f64, p], ctypes.c_int),
        "dsa_latent_store": ([p, R, P, p, p], ctypes.c_int),
        "dsa_fused_norm_rope_store": ([p, i64, p, p, R, P, p, p, p, i64, i64, f64, f64, f64, f64, p], ctypes.c_int),
        "dsa_logits_stride": ([i32], i64),
        "dsa_logits_rows_per_chunk": ([i64, i64, i64], i64),
        "dsa_set_topk_direct_limit": ([i64], i64),
        "dsa_indexer_logits": ([p, p, p, R, P, p, p, i64, p], ctypes.c_int),
        "dsa_indexer_logits_mxfp4": ([p, p, p, R, P, p, p, i64, p], ctypes.c_int),
        "dsa_topk_workspace_size": ([i32, i64, i32], sz),
        "dsa_topk": ([p, i64, R, i32, p, p, sz, p], ctypes.c_int),
        "dsa_indexer_topk": ([p, p, p, R, P, p, p, i64, i32, p, p, sz, p], ctypes.c_int),
        "dsa_indexer_topk_mxfp4": ([p, p, p, R, P, p, p, i64, i32, p, p, sz, p], ctypes.c_int),
        "dsa_sparse_mla_workspace_size": ([i32, i32], sz),
        "dsa_sparse_mla_decode": ([p, R, P, p, p, i32, f32, p, p, p, sz, p], ctypes.c_int),
        "dsa_sparse_mla_prefill": ([p, R, P, p, p, i32, f32, p, p, p, sz, p], ctypes.c_int),
        "dsa_sparse_mla_decode_noalloc": ([p, R, P, p, p, i32, f32, p, p, p], ctypes.c_int),
        "dsa_probe_stream_read": ([p, i64, p, p], ctypes.c_int),
        "dsa_probe_gather_records": ([p, i64, i32, p, i64, p, p], ctypes.c_int),
        "dsa_check_device_errors": ([], ctypes.c_int),
    }
    for name, (args, ret) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ret
    return lib


_lib = _load()
EXPORTED = ("dsa_abi_version", "dsa_last_error", "dsa_layer_is_shared", "dsa_mtp_seed_width", "dsa_mtp_carry_allowed",
            "dsa_quant_fp8",
            "dsa_index_k_store", "dsa_index_k_store_mxfp4", "dsa_latent_store", "dsa_fused_norm_rope_store", "dsa_logits_stride",
            "dsa_logits_rows_per_chunk", "dsa_indexer_logits", "dsa_indexer_logits_mxfp4", "dsa_topk_workspace_size",
            "dsa_topk", "dsa_indexer_topk", "dsa_indexer_topk_mxfp4", "dsa_set_topk_direct_limit",
            "dsa_sparse_mla_workspace_size",
            "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill", "dsa_sparse_mla_decode_noalloc",
            "dsa_probe_stream_read", "dsa_probe_gather_records", "dsa_check_device_errors")


def _check(st: int):
    if st != 0:
        raise DsaError(st, (_lib.dsa_last_error() or b"").decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


@dataclass
class Rows:
    """Query rows / new tokens: int32 device tensors req, pos; `group` consecutive rows share a request."""
    req: torch.Tensor
    pos: torch.Tensor
    max_pos: int
    group: int = 1

    def c(self) -> _Rows:
        return _Rows(_ptr(self.req), _ptr(self.pos), int(self.pos.numel()), int(self.group), int(self.max_pos))


@dataclass
class Pages:
    """Page table (int32 device [num_reqs, pt_stride]) shared by both caches, and the pool size."""
    page_table: torch.Tensor
    num_pages: int

    def c(self) -> _Pages:
        pt = self.page_table
        return _Pages(_ptr(pt), int(pt.shape[1]), int(pt.shape[0]), int(self.num_pages))


def abi_version() -> int:
    return _lib.dsa_abi_version()


def dsa_layer_is_shared(layer_id: int, indexer_types: str | None = None, cli_factor: int = 1,
                        topk_pattern: str | None = None, topk_freq: int = 1, skip_topk_offset: int = 2) -> bool:
    t = indexer_types.encode() if indexer_types is not None else None
    pat = topk_pattern.encode() if topk_pattern is not None else None
    rule = _Rule(t, len(t) if t else 0, cli_factor, pat, len(pat) if pat else 0, topk_freq, skip_topk_offset)
    r = _lib.dsa_layer_is_shared(ctypes.byref(rule), layer_id)
    if r < 0:
        raise DsaError(1, "invalid layer rule")
    return bool(r)


def dsa_quant_fp8(x, y, scale, stream=None):
    _check(_lib.dsa_quant_fp8(_ptr(x), x.numel() // 128, _ptr(y), _ptr(scale), _stream(stream)))


def dsa_mtp_seed_width(index_topk: int = 2048, index_kpool: int = 1) -> int:
    return int(_lib.dsa_mtp_seed_width(index_topk, index_kpool))


def dsa_mtp_carry_allowed(eagle_topk: int) -> int:
    return int(_lib.dsa_mtp_carry_allowed(eagle_topk))


def dsa_index_k_store(k, rows: Rows, pages: Pages, index_cache, ln_eps=1e-6, rope_theta=10000.0, stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_index_k_store(_ptr(k), ctypes.byref(r), ctypes.byref(p), _ptr(index_cache), ln_eps,
                                  rope_theta, _stream(stream)))


def dsa_index_k_store_mxfp4(k, rows: Rows, pages: Pages, index_cache, ln_eps=1e-6, rope_theta=10000.0,
                            stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_index_k_store_mxfp4(_ptr(k), ctypes.byref(r), ctypes.byref(p), _ptr(index_cache), ln_eps,
                                        rope_theta, _stream(stream)))


def dsa_latent_store(kv, rows: Rows, pages: Pages, latent_cache, stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_latent_store(_ptr(kv), ctypes.byref(r), ctypes.byref(p), _ptr(latent_cache), _stream(stream)))


def dsa_fused_norm_rope_store(kv, rows: Rows, pages: Pages, latent_cache, index_cache=None, k_idx=None, gamma=None,
                              q_pe=None, rms_eps=1e-6, ln_eps=1e-6, rope_theta=10000.0, index_rope_theta=10000.0,
                              stream=None):
    """kv: bf16 (int16) [n, >=576] view with unit column stride (its row stride is passed);
    q_pe: None or a [n, 64, 64] view with unit last stride (e.g. q[:, :, 512:]), rotated in place."""
    r, p = rows.c(), pages.c()
    if kv.dim() != 2 or kv.stride(1) != 1:
        raise ValueError("kv must be a 2-D view with unit column stride")
    qrs = qhs = 0
    if q_pe is not None:
        if q_pe.dim() != 3 or q_pe.shape[1:] != (64, 64) or q_pe.stride(2) != 1:
            raise ValueError("q_pe must be a [n, 64, 64] view with unit last stride")
        qrs, qhs = q_pe.stride(0), q_pe.stride(1)
    _check(_lib.dsa_fused_norm_rope_store(_ptr(kv), kv.stride(0), _ptr(gamma), _ptr(k_idx), ctypes.byref(r),
                                          ctypes.byref(p), _ptr(latent_cache), _ptr(index_cache), _ptr(q_pe), qrs,
                                          qhs, rms_eps, ln_eps, rope_theta, index_rope_theta, _stream(stream)))


def dsa_logits_stride(max_pos: int) -> int:
    return _lib.dsa_logits_stride(max_pos)


def dsa_logits_rows_per_chunk(num_rows: int, row_bytes: int, budget_bytes: int) -> int:
    return _lib.dsa_logits_rows_per_chunk(num_rows, row_bytes, budget_bytes)


def dsa_indexer_logits(q8, q_scale, w, rows: Rows, pages: Pages, index_cache, logits, stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_indexer_logits(_ptr(q8), _ptr(q_scale), _ptr(w), ctypes.byref(r), ctypes.byref(p),
                                   _ptr(index_cache), _ptr(logits), logits.shape[-1], _stream(stream)))


def dsa_indexer_logits_mxfp4(q8, q_scale, w, rows: Rows, pages: Pages, index_cache, logits, stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_indexer_logits_mxfp4(_ptr(q8), _ptr(q_scale), _ptr(w), ctypes.byref(r), ctypes.byref(p),
                                         _ptr(index_cache), _ptr(logits), logits.shape[-1], _stream(stream)))


def dsa_set_topk_direct_limit(max_scores: int) -> int:
    """Sets the score-array size up to which the fused indexer + top-k takes the radix path
    directly; returns the previous limit (a negative argument only reads it)."""
    return int(_lib.dsa_set_topk_direct_limit(max_scores))


def dsa_topk_workspace_size(R: int, stride: int, k: int) -> int:
    return _lib.dsa_topk_workspace_size(R, stride, k)


def dsa_topk(logits, rows: Rows, k: int, idx, ws, stream=None):
    r = rows.c()
    _check(_lib.dsa_topk(_ptr(logits), logits.shape[-1], ctypes.byref(r), k, _ptr(idx), _ptr(ws),
                         0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dsa_indexer_topk(q8, q_scale, w, rows: Rows, pages: Pages, index_cache, logits, k: int, idx, ws, stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_indexer_topk(_ptr(q8), _ptr(q_scale), _ptr(w), ctypes.byref(r), ctypes.byref(p),
                                 _ptr(index_cache), _ptr(logits), logits.shape[-1], k, _ptr(idx), _ptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dsa_indexer_topk_mxfp4(q8, q_scale, w, rows: Rows, pages: Pages, index_cache, logits, k: int, idx, ws,
                           stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_indexer_topk_mxfp4(_ptr(q8), _ptr(q_scale), _ptr(w), ctypes.byref(r), ctypes.byref(p),
                                       _ptr(index_cache), _ptr(logits), logits.shape[-1], k, _ptr(idx), _ptr(ws),
                                       0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def dsa_sparse_mla_workspace_size(R: int, k: int) -> int:
    return _lib.dsa_sparse_mla_workspace_size(R, k)


def _mla(fn, q, rows, pages, latent_cache, idx, sm_scale, out, lse, ws, stream):
    r, p = rows.c(), pages.c()
    _check(fn(_ptr(q), ctypes.byref(r), ctypes.byref(p), _ptr(latent_cache), _ptr(idx), idx.shape[-1],
              sm_scale, _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
              _stream(stream)))


def dsa_sparse_mla_decode(q, rows: Rows, pages: Pages, latent_cache, idx, out, lse=None, ws=None,
                          sm_scale=1.0 / 16.0, stream=None):
    _mla(_lib.dsa_sparse_mla_decode, q, rows, pages, latent_cache, idx, sm_scale, out, lse, ws, stream)


def dsa_sparse_mla_prefill(q, rows: Rows, pages: Pages, latent_cache, idx, out, lse=None, ws=None,
                           sm_scale=1.0 / 16.0, stream=None):
    _mla(_lib.dsa_sparse_mla_prefill, q, rows, pages, latent_cache, idx, sm_scale, out, lse, ws, stream)


def dsa_sparse_mla_decode_noalloc(q, rows: Rows, pages: Pages, latent_cache, idx, out, lse=None, sm_scale=1.0 / 16.0,
                                  stream=None):
    r, p = rows.c(), pages.c()
    _check(_lib.dsa_sparse_mla_decode_noalloc(_ptr(q), ctypes.byref(r), ctypes.byref(p), _ptr(latent_cache), _ptr(idx),
                                              idx.shape[-1], sm_scale, _ptr(out), _ptr(lse), _stream(stream)))


def dsa_probe_stream_read(buf, sink, stream=None):
    _check(_lib.dsa_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def dsa_probe_gather_records(pool, rec_bytes: int, ids, sink, stream=None):
    nbytes = pool.numel() * pool.element_size()
    _check(_lib.dsa_probe_gather_records(_ptr(pool), nbytes // rec_bytes, rec_bytes, _ptr(ids), ids.numel(), _ptr(sink),
                                         _stream(stream)))


def dsa_check_device_errors():
    _check(_lib.dsa_check_device_errors())
