"""GPU parity of the MXFP4 index-K variant (68 B per token; "GLM-5.3 推理全链路(十一)", the
paragraph on vLLM's two indexer-cache formats) against the CPU oracle on the same seeded inputs:
the store byte for byte, the logits within the indexer tolerance, and the fused indexer + top-k
equal to the separate calls and to the oracle's sets."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import LN_EPS, THETA, all_tokens, assert_logits_close, queries, raw_k, topk_path, topk_sets_match

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402

DEV = "cuda"
MX_PAGE = 64 * 68


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy()


def _announce(name):
    print(f"\n[gpu] {name}", flush=True)


def oracle_mx_cache(w):
    req, pos = all_tokens(w)
    cache = np.zeros((w.num_pages, MX_PAGE), np.uint8)
    orc.index_k_store_mxfp4(raw_k(w), req, pos, w.page_table, cache, LN_EPS, THETA)
    return cache


def gpu_mx_cache(w):
    req, pos = all_tokens(w)
    cache = torch.zeros((w.num_pages, MX_PAGE), dtype=torch.uint8, device=DEV)
    tok = dsa.Rows(dev(req), dev(pos), int(pos.max()), 1)
    pages = dsa.Pages(dev(w.page_table), w.num_pages)
    dsa.dsa_index_k_store_mxfp4(dev(raw_k(w).view(np.int16)), tok, pages, cache, LN_EPS, THETA)
    torch.cuda.synchronize()
    return cache


def rows_pages(w):
    return (dsa.Rows(dev(w.row_req), dev(w.row_pos), w.max_pos, w.rows_per_req),
            dsa.Pages(dev(w.page_table), w.num_pages))


def q_inputs(w):
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    return q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32), wt


@pytest.mark.parametrize("cid", [0, 1, 2])
def test_mxfp4_store_bit_exact(cid):
    _announce(f"mxfp4 store c{cid}")
    w = gi.config(cid, "small")
    got = host(gpu_mx_cache(w))
    ref = oracle_mx_cache(w)
    diff = np.argwhere(got != ref)
    assert len(diff) == 0, f"{len(diff)} MXFP4 index-K bytes differ, first at {diff[:5].tolist()}"
    dsa.dsa_check_device_errors()


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_mxfp4_logits_stage(cid):
    _announce(f"mxfp4 logits c{cid}")
    w = gi.config(cid, "small")
    cache = oracle_mx_cache(w)
    q8, qs, wt = q_inputs(w)
    ref = orc.indexer_logits_mxfp4(q8, qs, wt, w.row_req, w.row_pos, w.page_table, cache)
    rows, pages = rows_pages(w)
    logits = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_logits_mxfp4(dev(q8), dev(qs), dev(wt), rows, pages, dev(cache), logits)
    torch.cuda.synchronize()
    assert_logits_close(host(logits), ref)


@pytest.mark.parametrize("path", ["direct", "filtered"])
@pytest.mark.parametrize("cid", [0, 1, 2])
def test_mxfp4_fused_topk(cid, path):
    _announce(f"mxfp4 fused indexer+topk c{cid}, {path} path")
    w = gi.config(cid, "small")
    cache = gpu_mx_cache(w)
    q8, qs, wt = q_inputs(w)
    rows, pages = rows_pages(w)
    stride = orc.logits_stride(w.max_pos)
    logits = torch.empty((w.R, stride), dtype=torch.float32, device=DEV)
    idx = torch.full((w.R, 2048), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(dsa.dsa_topk_workspace_size(w.R, stride, 2048), dtype=torch.uint8, device=DEV)
    dq8, dqs, dwt = dev(q8), dev(qs), dev(wt)
    with topk_path(path):
        dsa.dsa_indexer_topk_mxfp4(dq8, dqs, dwt, rows, pages, cache, logits, 2048, idx, ws)
    torch.cuda.synchronize()
    fused = host(idx).copy()
    dsa.dsa_indexer_logits_mxfp4(dq8, dqs, dwt, rows, pages, cache, logits)
    dsa.dsa_topk(logits, rows, 2048, idx, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), fused)              # same scores, same exact selection
    ref_lg = orc.indexer_logits_mxfp4(q8, qs, wt, w.row_req, w.row_pos, w.page_table, host(cache))
    ridx, kth = orc.topk(ref_lg, w.row_pos, 2048)
    topk_sets_match(fused, ridx, ref_lg, kth)


def test_mxfp4_store_special_keys():
    """Keys whose LayerNorm output is all zero (a constant raw key: scale byte 127, zero codes),
    very large and very small raw keys, and exact powers of two: bit-exact against the oracle."""
    _announce("mxfp4 store, special keys")
    n = 64
    rng = np.random.default_rng(61)
    raw = rng.standard_normal((n, 128))
    raw[0] = 3.0                                  # constant: LayerNorm gives zeros
    raw[1] *= 1e30
    raw[2] *= 1e-30
    raw[3] = np.where(np.arange(128) % 2 == 0, 4.0, -4.0)
    raw[4, :] = 0.0
    raw[4, 7] = 1.0                               # one spike
    k = orc.bf16_from_double(raw)
    pos = np.arange(n, dtype=np.int32)
    pt = np.array([[0]], np.int32)
    ref = np.zeros((1, MX_PAGE), np.uint8)
    orc.index_k_store_mxfp4(k, np.zeros(n, np.int32), pos, pt, ref, LN_EPS, THETA)
    cache = torch.zeros((1, MX_PAGE), dtype=torch.uint8, device=DEV)
    tok = dsa.Rows(dev(np.zeros(n, np.int32)), dev(pos), n - 1, 1)
    dsa.dsa_index_k_store_mxfp4(dev(k.view(np.int16)), tok, dsa.Pages(dev(pt), 1), cache, LN_EPS, THETA)
    torch.cuda.synchronize()
    got = host(cache)
    diff = np.argwhere(got != ref)
    assert len(diff) == 0, f"{len(diff)} bytes differ, first at {diff[:5].tolist()}"
    assert got[0, 4096] == 127 and not got[0, :64].any()     # the constant key


# ----------------------------------------------------------------------------- full size
def oracle_mx_cache_of(w, b, overrides=None):
    """Request b's MXFP4 index-K cache alone, in a compact pool (page i of the request is pool
    page i; scores do not depend on page placement)."""
    L = int(w.ctx[b])
    npg = (L + 63) // 64
    pt = np.arange(npg, dtype=np.int32)[None, :]
    k = gi.normal_bf16(w.seed, gi.T_RAW_K, int(w.token_base[b]) * 128, L * 128).reshape(L, 128)
    for p, v in (overrides or {}).items() if b == 0 else ():
        k[p] = v
    cache = np.zeros((npg, MX_PAGE), np.uint8)
    orc.index_k_store_mxfp4(k, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), pt, cache, LN_EPS, THETA)
    return cache, pt


def _full_size_mx(w, sample_reqs, overrides=None, path=None):
    """The benchmark's launch configuration on the whole batch (every request stored, scored and
    selected on the GPU), checked against the oracle on the sampled requests' rows: logits
    element-wise, the fused and the separate selections against the oracle's sets."""
    from parity import row_queries
    from sparse_attention_store_amd.workload import DeviceLayer
    L = DeviceLayer(w, latent_layers=[], k_overrides=overrides)
    cache = L.build_mxfp4_index(0)
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    with topk_path(path):
        dsa.dsa_indexer_topk_mxfp4(L.q8, L.qs, L.w_head, L.rows, L.pages, cache, L.logits, 2048, L.idx, L.ws_topk)
    torch.cuda.synchronize()
    fused = host(L.idx).copy()
    dsa.dsa_indexer_logits_mxfp4(L.q8, L.qs, L.w_head, L.rows, L.pages, cache, L.logits)
    torch.cuda.synchronize()
    n_same = n_rows = 0
    for b in sample_reqs:
        rs = np.where(w.row_req == b)[0]
        mx, pt = oracle_mx_cache_of(w, b, overrides)
        q, wt, _ = row_queries(w, rs, [])
        q8, qs = orc.quant_fp8(q.reshape(-1, 128))
        pos = w.row_pos[rs]
        ref = orc.indexer_logits_mxfp4(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, np.zeros(len(rs), np.int32),
                                       pos, pt, mx)
        got = host(L.logits[torch.as_tensor(rs, device=DEV)])
        ow = ref.shape[1]
        assert_logits_close(got[:, :ow], ref)
        assert np.all(np.isneginf(got[:, ow:]))
        ridx, kth = orc.topk(ref, pos, 2048)
        topk_sets_match(fused[rs], ridx, ref, kth)
        n_same += sum(set(fused[r]) == set(ridx[i]) for i, r in enumerate(rs))
        n_rows += len(rs)
    # the separate radix top-k over the same GPU scores selects exactly what the fused call did
    dsa.dsa_topk(L.logits, L.rows, 2048, L.idx, L.ws_topk)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx), fused)
    dsa.dsa_check_device_errors()
    del L, cache
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return n_same, n_rows


def test_mxfp4_full_c2_verify_128k_sampled_requests():
    _announce("mxfp4 full size c2: 64 x 6 rows at 128K, 6 sampled requests")
    w = gi.config(2, "full")
    n_same, n = _full_size_mx(w, [0, 1, 31, 32, 62, 63])
    assert n_same >= 0.9 * n, f"only {n_same}/{n} rows have the oracle's exact set"


@pytest.mark.parametrize("path", ["direct", "filtered"])
def test_mxfp4_full_c3_long_1m(path):
    _announce(f"mxfp4 full size c3: 1 request at 1M context (needle keys stored as MXFP4), {path} top-k")
    from parity import needle_overrides
    w = gi.config(3, "full")
    _full_size_mx(w, [0], needle_overrides(w), path)    # the set differs only at near-ties
