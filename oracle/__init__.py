"""CPU oracle for the DSA attention-layer hot path.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; the product package never imports it, and it shares
no code with the HIP path.

The arithmetic lives in ``dsa_oracle.c`` (plain C, fp64); this module builds it with gcc,
loads it through ctypes and adds the pages' byte accounting as plain formulas.

Pages cited (title, section):
  [IDXC] "GLM-5.3 推理全链路(十一): 索引器缓存的跨层读写"
  [REQ]  "GLM-5.3 推理全链路(一): 一个请求在 SGLang 里经过哪些算子、哪些通信"
  [VLLM] "vLLM 推理链路概览: 以 GLM-5.2 为例"

Every function is pinned by a CPU test (tests/test_oracle_*.py) to something other than
itself: brute force, closed forms, invariants, or numbers printed on the pages.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")

IDX_PAGE_BYTES = 8448
IDX_MXFP4_PAGE_BYTES = 64 * 68
LAT_PAGE_BYTES = 64 * 656


def build() -> str:
    """Compile the oracle (gcc, -O2 -ffp-contract=off so no fused multiply-add changes rounding)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Wextra", os.path.join(HERE, "dsa_oracle.c"), "-o", LIB, "-lm"]
    subprocess.check_call(cmd)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        p, i64, i32, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        sig = {
            "orc_fp8_encode_array": [p, i64, p, ctypes.c_int],
            "orc_fp8_decode_array": [p, i64, p],
            "orc_bf16_from_double_array": [p, i64, p],
            "orc_ue8m0_array": [p, i64, p],
            "orc_ln_rope_array": [p, p, i64, d, d, ctypes.c_int, ctypes.c_int, p],
            "orc_quant_fp8": [p, i64, p, p],
            "orc_index_k_store": [p, p, p, i64, p, i64, p, d, d, p],
            "orc_latent_store": [p, p, p, i64, p, i64, p],
            "orc_fused_norm_rope_store": [p, i64, p, p, p, p, i64, p, i64, p, p, p, i64, i64, d, d, d, d],
            "orc_indexer_logits": [p, p, p, p, p, i64, p, i64, p, p, i64],
            "orc_topk": [p, i64, p, i64, i32, p, p],
            "orc_sparse_mla": [p, p, p, i64, p, i64, p, p, i32, d, p, p],
            "orc_layer_is_shared": [ctypes.c_char_p, i32, i32, ctypes.c_char_p, i32, i32, i32, i32],
            "orc_fp4_encode_array": [p, i64, p, ctypes.c_int],
            "orc_fp4_decode_array": [p, i64, p],
            "orc_ue8m0_fp4_array": [p, i64, p],
            "orc_index_k_store_mxfp4": [p, p, p, i64, p, i64, p, d, d],
            "orc_indexer_logits_mxfp4": [p, p, p, p, p, i64, p, i64, p, p, i64],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int if name == "orc_layer_is_shared" else None
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


# ----------------------------------------------------------------------------- codecs
def fp8_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_fp8_decode_array(c.ctypes.data, c.size, out.ctypes.data)
    return out


def fp8_encode(x, brute: bool = False) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().orc_fp8_encode_array(x.ctypes.data, x.size, out.ctypes.data, int(brute))
    return out


def ue8m0(amax) -> np.ndarray:
    a = _c(amax, np.float64)
    out = np.empty(a.shape, np.float64)
    lib().orc_ue8m0_array(a.ctypes.data, a.size, out.ctypes.data)
    return out


def fp4_decode(codes) -> np.ndarray:
    """MXFP4 element codes (the low 4 bits of each byte) -> values."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_fp4_decode_array(c.ctypes.data, c.size, out.ctypes.data)
    return out


def fp4_encode(x, brute: bool = False) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().orc_fp4_encode_array(x.ctypes.data, x.size, out.ctypes.data, int(brute))
    return out


def ue8m0_fp4(amax) -> np.ndarray:
    a = _c(amax, np.float64)
    out = np.empty(a.shape, np.float64)
    lib().orc_ue8m0_fp4_array(a.ctypes.data, a.size, out.ctypes.data)
    return out


def bf16_from_double(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_from_double_array(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_to_double(h) -> np.ndarray:
    return (_c(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ln_rope(x, pos, eps: float = 1e-6, theta: float = 10000.0, ln: bool = True,
            inverse: bool = False) -> np.ndarray:
    """LayerNorm (optional) then interleaved RoPE on dims 0..63, per 128-vector."""
    x = _c(x, np.float64).reshape(-1, 128)
    pos = _c(np.broadcast_to(pos, (x.shape[0],)), np.int64)
    out = np.empty_like(x)
    lib().orc_ln_rope_array(x.ctypes.data, pos.ctypes.data, x.shape[0], eps, theta, int(ln),
                            int(inverse), out.ctypes.data)
    return out


# ----------------------------------------------------------------------------- stages
def quant_fp8(x_bf16):
    """[n, 128] bf16 bits -> (fp8 codes [n, 128], fp32 scales [n])."""
    x = _c(x_bf16, np.uint16).reshape(-1, 128)
    codes = np.empty(x.shape, np.uint8)
    scale = np.empty(x.shape[0], np.float32)
    lib().orc_quant_fp8(x.ctypes.data, x.shape[0], codes.ctypes.data, scale.ctypes.data)
    return codes, scale


def index_k_store(k_bf16, req, pos, page_table, cache, eps=1e-6, theta=10000.0, want_pre=False):
    """Writes into ``cache`` (uint8 [pages, 8448]) in place; returns pre-rounding y/scale if asked."""
    k = _c(k_bf16, np.uint16).reshape(-1, 128)
    req, pos = _c(req, np.int32), _c(pos, np.int32)
    pt = _c(page_table, np.int32)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.shape[-1] == IDX_PAGE_BYTES
    pre = np.full(k.shape, np.nan) if want_pre else None
    lib().orc_index_k_store(k.ctypes.data, req.ctypes.data, pos.ctypes.data, k.shape[0],
                            pt.ctypes.data, pt.shape[1], cache.ctypes.data, eps, theta, _ptr(pre))
    return pre


def index_k_store_mxfp4(k_bf16, req, pos, page_table, cache, eps=1e-6, theta=10000.0):
    """Writes into ``cache`` (uint8 [pages, 4352], the MXFP4 index-K layout) in place."""
    k = _c(k_bf16, np.uint16).reshape(-1, 128)
    req, pos = _c(req, np.int32), _c(pos, np.int32)
    pt = _c(page_table, np.int32)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.shape[-1] == IDX_MXFP4_PAGE_BYTES
    lib().orc_index_k_store_mxfp4(k.ctypes.data, req.ctypes.data, pos.ctypes.data, k.shape[0],
                                  pt.ctypes.data, pt.shape[1], cache.ctypes.data, eps, theta)


def latent_store(kv_bf16, req, pos, page_table, cache):
    kv = _c(kv_bf16, np.uint16).reshape(-1, 576)
    req, pos, pt = _c(req, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous and cache.shape[-1] == LAT_PAGE_BYTES
    lib().orc_latent_store(kv.ctypes.data, req.ctypes.data, pos.ctypes.data, kv.shape[0],
                           pt.ctypes.data, pt.shape[1], cache.ctypes.data)


def fused_norm_rope_store(kv_bf16, req, pos, page_table, latent_cache, index_cache=None, k_idx=None,
                          gamma=None, q=None, q_off=0, rms_eps=1e-6, ln_eps=1e-6, theta=10000.0,
                          index_theta=10000.0, kv_off=0):
    """RMSNorm(kv[:, o:o+512]) * gamma and RoPE(kv[:, o+512:o+576]) (o = ``kv_off``) into the
    656-B records of ``latent_cache``; the index-K entries of ``k_idx`` into ``index_cache``
    when both are given; ``q`` (uint16 [n, 64, W], C-contiguous, nullable) has its 64 rope dims
    per head at ``q_off`` rotated in place.  ``kv_bf16`` is [n, S] (S is the row stride)."""
    kv = _c(kv_bf16, np.uint16)
    assert kv.ndim == 2 and 0 <= kv_off and kv_off + 576 <= kv.shape[1]
    n = kv.shape[0]
    req, pos, pt = _c(req, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    assert latent_cache.dtype == np.uint8 and latent_cache.flags.c_contiguous
    assert latent_cache.shape[-1] == LAT_PAGE_BYTES
    g = None if gamma is None else _c(gamma, np.uint16)
    ki = None if k_idx is None else _c(k_idx, np.uint16).reshape(-1, 128)
    if index_cache is not None:
        assert index_cache.dtype == np.uint8 and index_cache.flags.c_contiguous
        assert index_cache.shape[-1] == IDX_PAGE_BYTES
    qp, qrs, qhs = None, 0, 0
    if q is not None:
        assert q.dtype == np.uint16 and q.flags.c_contiguous and q.shape[:2] == (n, 64)
        assert 0 <= q_off and q_off + 64 <= q.shape[2]
        qp = q.ctypes.data + 2 * q_off
        qrs, qhs = 64 * q.shape[2], q.shape[2]
    lib().orc_fused_norm_rope_store(kv.ctypes.data + 2 * kv_off, kv.shape[1], _ptr(g), _ptr(ki), req.ctypes.data,
                                    pos.ctypes.data, n, pt.ctypes.data, pt.shape[1], latent_cache.ctypes.data,
                                    _ptr(index_cache), qp, qrs, qhs, rms_eps, ln_eps, theta, index_theta)


def logits_stride(max_pos: int) -> int:
    """Row stride of the logits buffer: visible length rounded up to 256 elements
    ([IDXC] §临时缓冲:logits 矩阵, MQA_LOGITS_ROW_ALIGN_ELEMS = 256)."""
    return ((max_pos + 1 + 255) // 256) * 256


def indexer_logits(q8, q_scale, w, req, pos, page_table, cache, stride=None):
    q8 = _c(q8, np.uint8).reshape(-1, 32, 128)
    R = q8.shape[0]
    qs, w = _c(q_scale, np.float32).reshape(R, 32), _c(w, np.float32).reshape(R, 32)
    req, pos, pt = _c(req, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    if stride is None:
        stride = logits_stride(int(pos.max()))
    out = np.empty((R, stride), np.float32)
    lib().orc_indexer_logits(q8.ctypes.data, qs.ctypes.data, w.ctypes.data, req.ctypes.data,
                             pos.ctypes.data, R, pt.ctypes.data, pt.shape[1],
                             _c(cache, np.uint8).ctypes.data, out.ctypes.data, stride)
    return out


def indexer_logits_mxfp4(q8, q_scale, w, req, pos, page_table, cache, stride=None):
    q8 = _c(q8, np.uint8).reshape(-1, 32, 128)
    R = q8.shape[0]
    qs, w = _c(q_scale, np.float32).reshape(R, 32), _c(w, np.float32).reshape(R, 32)
    req, pos, pt = _c(req, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    if stride is None:
        stride = logits_stride(int(pos.max()))
    out = np.empty((R, stride), np.float32)
    lib().orc_indexer_logits_mxfp4(q8.ctypes.data, qs.ctypes.data, w.ctypes.data, req.ctypes.data,
                                   pos.ctypes.data, R, pt.ctypes.data, pt.shape[1],
                                   _c(cache, np.uint8).ctypes.data, out.ctypes.data, stride)
    return out


def topk(logits, pos, k: int = 2048):
    """Returns (idx [R, k] ascending with -1 tail, kth score [R] or NaN)."""
    lg = _c(logits, np.float32)
    pos = _c(pos, np.int32)
    R = lg.shape[0]
    idx = np.empty((R, k), np.int32)
    kth = np.empty(R, np.float32)
    lib().orc_topk(lg.ctypes.data, lg.shape[1], pos.ctypes.data, R, k, idx.ctypes.data, kth.ctypes.data)
    return idx, kth


def sparse_mla(q_bf16, req, pos, page_table, latent_cache, idx, sm_scale=1.0 / 16.0):
    q = _c(q_bf16, np.uint16).reshape(-1, 64, 576)
    R = q.shape[0]
    idx = _c(idx, np.int32).reshape(R, -1)
    req, pos, pt = _c(req, np.int32), _c(pos, np.int32), _c(page_table, np.int32)
    out = np.empty((R, 64, 512), np.uint16)
    lse = np.empty((R, 64), np.float32)
    lib().orc_sparse_mla(q.ctypes.data, req.ctypes.data, pos.ctypes.data, R, pt.ctypes.data,
                         pt.shape[1], _c(latent_cache, np.uint8).ctypes.data, idx.ctypes.data,
                         idx.shape[1], sm_scale, out.ctypes.data, lse.ctypes.data)
    return out, lse


def layer_is_shared(layer_id: int, indexer_types=None, cli_factor: int = 1, pattern=None,
                    topk_freq: int = 1, skip_topk_offset: int = 2) -> bool:
    """indexer_types: list of "full"/"shared" strings, or a string of 'F'/'S'."""
    t = None
    if indexer_types is not None:
        t = "".join(("S" if x == "shared" else "F") if len(x) > 1 else x for x in indexer_types).encode()
    pat = pattern.encode() if pattern is not None else None
    r = lib().orc_layer_is_shared(t, len(t) if t else 0, cli_factor, pat, len(pat) if pat else 0,
                                  topk_freq, skip_topk_offset, layer_id)
    if r < 0:
        raise ValueError("invalid layer rule")
    return bool(r)


# ----------------------------------------------------------------------------- byte accounting
# [IDXC] §索引器缓存里存的是什么 (page width), §读的字节数 (read), §读的带宽 (time model),
# 一笔写 (write), §临时缓冲:logits 矩阵, 判断四 (pool memory), 读取路径里的两条"非缓存"字节.
def index_k_bytes_per_token(head_dim: int = 128, quant_block: int = 128) -> int:
    return head_dim + head_dim // quant_block * 4


def index_k_page_bytes(page_size: int = 64, index_kpool: int = 1, head_dim: int = 128,
                       quant_block: int = 128) -> int:
    return page_size // index_kpool * index_k_bytes_per_token(head_dim, quant_block)


def latent_bytes_per_token(latent: int = 512, rope: int = 64, block: int = 128) -> int:
    """Record layout read of the pages' 656 B: scaled fp8 latent blocks + bf16 rope tail."""
    return latent + (latent // block) * 4 + rope * 2


def read_bytes_per_full_layer(L: int) -> int:
    return index_k_bytes_per_token() * L


def read_bytes_per_step(L: int, n_full: int = 21) -> int:
    return n_full * read_bytes_per_full_layer(L)


def write_bytes_per_step(n_tokens: int = 1, n_full: int = 21) -> int:
    return n_full * index_k_bytes_per_token() * n_tokens


def index_read_seconds(b: int, L: int, hbm_bytes_per_s: float, n_full: int = 21) -> float:
    return n_full * index_k_bytes_per_token() * b * L / hbm_bytes_per_s


def mtp_seed_width(index_topk: int = 2048, index_kpool: int = 1) -> int:
    """Width of the top-k seed an MTP draft iteration carries across its steps:
    index_topk + index_kpool - 1 ([IDXC] §优化三:MTP 迭代内复用 topk)."""
    return index_topk + index_kpool - 1


def mtp_carry_allowed(eagle_topk: int) -> bool:
    """The carry is valid only for a single draft chain ([IDXC] §优化三: top-k > 1 reorders rows)."""
    return eagle_topk == 1


def mtp_carry_saved_read_bytes(L: int, draft_steps: int = 5) -> int:
    """Indexer-cache reads the carry saves per MTP iteration: all draft steps but the first skip
    scoring the MTP layer's own cache ([IDXC] §优化三)."""
    return (draft_steps - 1) * index_k_bytes_per_token() * L


def mtp_carry_saved_fraction(draft_steps: int = 5, n_full: int = 21) -> float:
    """The saving relative to the main model's indexer reads per step (n_full x 132 L)."""
    return mtp_carry_saved_read_bytes(1, draft_steps) / read_bytes_per_step(1, n_full)


def chunked_prefill_indexer_read_bytes(L: int, rows_per_read: int, n_full: int = 21) -> int:
    """Index-K bytes the prefill of an L-token prompt reads when each block of `rows_per_read`
    consecutive query rows reads the keys visible to its last row once, 132 B per token, per
    full layer.  A kernel that reads the cache once per 32K-row chunk reads `rows_per_read` =
    32768's worth.  The read granularity is an argument with no default: the page's 1M prefill
    figure ([IDXC], the cross-layer section: about 47 TB, an accounting the page calls
    simplified) does not say how often a key is read, so no value of it is the page's.  The
    formula is pinned by its two limits (one row per block: every row reads its own prefix; one
    block: one read of the prompt) and by brute force on a tiny prompt."""
    n = (L + rows_per_read - 1) // rows_per_read
    return n_full * index_k_bytes_per_token() * sum(min(L, (b + 1) * rows_per_read) for b in range(n))


def chunked_prefill_indexer_flops(L: int = 1 << 20, n_full: int = 21, heads: int = 32, dim: int = 128) -> int:
    """Indexer scoring work of an L-token prefill: row i scores its i + 1 visible keys with
    `heads` dot products of `dim` dims (2 flops per multiply-add), per full layer."""
    return n_full * heads * dim * 2 * L * (L + 1) // 2


def logits_bytes(R: int, L: int) -> int:
    return 4 * R * math.ceil(L / 256) * 256


def logits_rows_per_chunk(num_rows: int, row_bytes: int, budget_bytes: int):
    if num_rows * row_bytes <= budget_bytes:
        return None
    rows = max(budget_bytes // max(row_bytes, 1), 1)
    return int(rows) if rows < num_rows else None


def index_pool_bytes(n_full: int, capacity_tokens: int) -> int:
    return n_full * index_k_bytes_per_token() * capacity_tokens


def indexer_q_bytes_per_token(heads: int = 32, head_dim: int = 128, block: int = 128) -> int:
    return heads * head_dim + heads * (head_dim // block) * 4


def block_table_bytes(L: int, page_size: int = 64) -> int:
    return 4 * math.ceil(L / page_size)
