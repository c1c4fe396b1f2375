"""Shared pieces of the GPU parity tests: oracle-side construction of a workload's caches and
expected outputs (host, from the seeded generator + the oracle only), and the comparison
rules with their tolerances.

Tolerances (the stated parity bar):
  logits     |g - r| <= 1e-3 |r| + 1e-5 * mean_row(|r|)   (fp8 MFMA accumulation is not exact
             fp32; the relative 1e-3 is the bar, the tiny floor covers values near zero)
  top-k      sets equal except positions whose oracle score lies within 1e-3 |tau| of the
             row's k-th score tau
  attention  |g - r| <= 2e-2 + 1e-2 |r|, element-wise on the bf16 outputs
  stores     bit-exact bytes
"""
from __future__ import annotations

import contextlib

import numpy as np

import dsa_inputs as gi
import oracle as orc

LN_EPS, THETA, SM = 1e-6, 10000.0, 1.0 / 16.0


def all_tokens(w: gi.Workload):
    req = np.concatenate([np.full(int(c), b, np.int32) for b, c in enumerate(w.ctx)])
    pos = np.concatenate([np.arange(int(c), dtype=np.int32) for c in w.ctx])
    return req, pos


def raw_k(w: gi.Workload, overrides=None):
    k = gi.normal_bf16(w.seed, gi.T_RAW_K, 0, w.total_tokens * 128).reshape(-1, 128)
    for p, v in (overrides or {}).items():
        k[p] = v                               # request 0: token index == position
    return k


def oracle_index_cache(w: gi.Workload, overrides=None):
    req, pos = all_tokens(w)
    cache = np.zeros((w.num_pages, 8448), np.uint8)
    orc.index_k_store(raw_k(w, overrides), req, pos, w.page_table, cache, LN_EPS, THETA)
    return cache


def oracle_latent_cache(w: gi.Workload, layer: int):
    req, pos = all_tokens(w)
    kv = gi.normal_bf16(w.seed, gi.T_LATENT0 + layer, 0, w.total_tokens * 576).reshape(-1, 576)
    cache = np.zeros((w.num_pages, 64 * 656), np.uint8)
    orc.latent_store(kv, req, pos, w.page_table, cache)
    return cache


def queries(w: gi.Workload, layers):
    R, r0, rt = w.R, w.row0, w.rows_total
    q = gi.normal_bf16(w.seed, gi.T_IDX_Q, r0 * 32 * 128, R * 32 * 128).reshape(R, 32, 128)
    wt = gi.uniform_f32(w.seed, gi.T_W, r0 * 32, R * 32, gi.w_scale()).reshape(R, 32)
    qm = {l: gi.normal_bf16(w.seed, gi.T_MLA_Q, (l * rt + r0) * 64 * 576, R * 64 * 576).reshape(R, 64, 576)
          for l in layers}
    return q, wt, qm


def needle_overrides(w: gi.Workload):
    """Raw keys for the planted needles of request 0: the inverse RoPE of the weighted query
    direction, centred and scaled so LayerNorm keeps it (built with the oracle's own RoPE)."""
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q[0])
    u = (orc.fp8_decode(q8) * qs[:, None] * wt[0][:, None]).sum(0)
    v = orc.ln_rope(np.repeat(u[None], len(w.needles), 0), w.needles, ln=False, inverse=True)
    v -= v.mean(1, keepdims=True)
    v *= np.sqrt(128) / np.linalg.norm(v, axis=1, keepdims=True)
    bits = orc.bf16_from_double(v)
    return {int(p): bits[i] for i, p in enumerate(w.needles)}


# ----------------------------------------------------------------------------- comparisons
def assert_logits_close(g, r, rows=None):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    fin = np.isfinite(r)
    assert np.array_equal(np.isfinite(g), fin), "masked (-inf) pattern differs"
    assert np.all(g[~fin] == r[~fin])
    mean = np.array([np.abs(r[i][fin[i]]).mean() if fin[i].any() else 0.0 for i in range(r.shape[0])])
    tol = 1e-3 * np.abs(r) + 1e-5 * mean[:, None]
    with np.errstate(invalid="ignore"):
        bad = fin & (np.abs(g - r) > tol)
    assert not bad.any(), f"{bad.sum()} logits out of tolerance; worst rel {np.max(np.abs(g - r)[fin] / (np.abs(r[fin]) + 1e-30)):.3g}"


def topk_sets_match(g_idx, r_idx, r_logits, kth, tol=1e-3):
    """Returns the number of rows whose sets differ (only allowed at near-ties)."""
    ndiff = 0
    for i in range(r_idx.shape[0]):
        a = set(int(x) for x in g_idx[i] if x >= 0)
        b = set(int(x) for x in r_idx[i] if x >= 0)
        assert len(a) == len([x for x in g_idx[i] if x >= 0]), f"row {i}: duplicate positions"
        assert len(a) == len(b), f"row {i}: {len(a)} selected vs {len(b)}"
        if a != b:
            ndiff += 1
            tau = float(kth[i])
            for p in a ^ b:
                assert abs(float(r_logits[i, p]) - tau) <= tol * abs(tau), \
                    f"row {i}: position {p} score {r_logits[i, p]} not a near-tie of tau {tau}"
        # -1 only as tail padding
        gi_ = np.asarray(g_idx[i])
        nv = (gi_ >= 0).sum()
        assert np.all(gi_[:nv] >= 0) and np.all(gi_[nv:] == -1)
    return ndiff


def bf16_to_f64(h):
    return orc.bf16_to_double(np.asarray(h).view(np.uint16))


def assert_attention_close(g_bits, r_bits, atol=2e-2, rtol=1e-2):
    g = bf16_to_f64(g_bits)
    r = bf16_to_f64(r_bits)
    assert g.shape == r.shape
    if g.size == 0:                      # no row left to compare (all differed at near-ties)
        return 0.0
    err = np.abs(g - r)
    tol = atol + rtol * np.abs(r)
    assert np.all(err <= tol), f"{(err > tol).sum()} outputs out of tolerance, max err {err.max():.3g}"
    return float(err.max())


# ----------------------------------------------------------------------------- one request at a time
# At full size the oracle works on sampled rows: it rebuilds only the sampled request's index-K
# cache and only the selected latent records, in a compact page pool of that request alone
# (page i of the request is pool page i; the result does not depend on page placement).
def request_pool(w: gi.Workload, b: int):
    npg = (int(w.ctx[b]) + 63) // 64
    return np.arange(npg, dtype=np.int32)[None, :], npg


def oracle_index_cache_of(w: gi.Workload, b: int, overrides=None):
    L = int(w.ctx[b])
    pt, npg = request_pool(w, b)
    k = gi.normal_bf16(w.seed, gi.T_RAW_K, int(w.token_base[b]) * 128, L * 128).reshape(L, 128)
    if b == 0:
        for p, v in (overrides or {}).items():
            k[p] = v
    cache = np.zeros((npg, 8448), np.uint8)
    orc.index_k_store(k, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), pt, cache, LN_EPS, THETA)
    return cache, pt


def oracle_latent_cache_of(w: gi.Workload, b: int, layer: int, positions):
    pt, npg = request_pool(w, b)
    positions = np.asarray(positions).ravel()
    sel = np.unique(positions[positions >= 0]).astype(np.int64)
    cache = np.zeros((npg, 64 * 656), np.uint8)
    if len(sel):
        flat = ((int(w.token_base[b]) + sel)[:, None] * 576 + np.arange(576)[None, :]).ravel()
        kv = gi.normal_bf16_at(w.seed, gi.T_LATENT0 + layer, flat).reshape(-1, 576)
        orc.latent_store(kv, np.zeros(len(sel), np.int32), sel.astype(np.int32), pt, cache)
    return cache, pt


def row_queries(w: gi.Workload, rows, layers):
    """Indexer q, head weights and MLA q of the given rows only (same values as queries())."""
    rows = [w.row0 + int(r) for r in rows]
    q = np.stack([gi.normal_bf16(w.seed, gi.T_IDX_Q, r * 32 * 128, 32 * 128) for r in rows]).reshape(-1, 32, 128)
    wt = np.stack([gi.uniform_f32(w.seed, gi.T_W, r * 32, 32, gi.w_scale()) for r in rows])
    qm = {l: np.stack([gi.normal_bf16(w.seed, gi.T_MLA_Q, (l * w.rows_total + r) * 64 * 576, 64 * 576)
                       for r in rows]).reshape(-1, 64, 576) for l in layers}
    return q, wt, qm


@contextlib.contextmanager
def topk_path(path):
    """Which path the fused indexer + top-k takes inside the block: "filtered" (sampled
    threshold, filter pass, exact selection over the candidates) for every call, "direct"
    (every score written, radix top-k) for every call, None the library's size rule."""
    from sparse_attention_store_amd import dsa
    if path is None:
        yield
        return
    prev = dsa.dsa_set_topk_direct_limit({"filtered": 0, "direct": 1 << 62}[path])
    try:
        yield
    finally:
        dsa.dsa_set_topk_direct_limit(prev)
