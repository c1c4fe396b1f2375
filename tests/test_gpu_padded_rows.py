"""GPU parity for padded query rows (pos < 0) and for reuse of the sparse-MLA workspace.

Padded rows are the normal case in captured decode buckets, whose batch is rounded up to a
fixed size ("GLM-5.3 推理全链路(一)", 第九阶段 细节四: CUDA Graph buckets).  The contract
(include/dsa.h): the logits of a padded row are -inf everywhere, its top-k is all -1, and
its attention output is 0 with lse = -inf.  Every check is element-wise against the oracle on
the same inputs; buffers are pre-filled with NaN so that an unwritten element shows.

The stream-K sparse MLA (256 rows or more) merges rows cut between two work-groups through
tag words in the workspace; these tests run it on a workspace pre-filled with stale small
integers, reuse one workspace across calls, and replay a captured graph of it several times.
"""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import (SM, all_tokens, assert_attention_close, assert_logits_close, oracle_index_cache,
                    oracle_latent_cache, queries, raw_k, topk_path, topk_sets_match)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402
from sparse_attention_store_amd.workload import DeviceLayer  # noqa: E402

DEV = "cuda"


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy()


def _announce(name):
    print(f"\n[gpu] {name}", flush=True)


def _padded(w, pad_rows):
    pos = w.row_pos.copy()
    pos[list(pad_rows)] = -1
    return pos


def _rows(w, pos):
    return dsa.Rows(dev(w.row_req), dev(pos), int(pos.max()), w.rows_per_req)


# (name, contexts, rows per request, padded rows): RG = 1 batches with idle rows, a group of six
# rows that is entirely padded, and groups that mix padded and live rows
PAD_CASES = [
    ("rg1_idle_rows", [3000, 2500, 5000, 4100, 2200], 1, [1, 3]),
    ("rg1_last_row_idle", [4097, 3333], 1, [1]),
    ("rg6_full_and_mixed", [3000, 4000, 5000, 2600], 6, list(range(6, 12)) + [14, 16, 23]),
    ("rg3_mixed", [2100, 4500], 3, [0, 5]),
]


@pytest.mark.parametrize("name,ctx,g,pad", PAD_CASES, ids=[c[0] for c in PAD_CASES])
@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
@pytest.mark.parametrize("path", ["direct", "filtered"])
def test_logits_and_topk_padded_rows(name, ctx, g, pad, fmt, path):
    _announce(f"padded rows: logits + top-k, {name}, {fmt}, {path} fused path")
    w = gi.make_decode(f"pad_{name}", gi.SEED_BASE + 80, ctx, rows_per_req=g)
    L = DeviceLayer(w)
    pos = _padded(w, pad)
    rows = _rows(w, pos)
    stride = dsa.dsa_logits_stride(int(pos.max()))
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    q8, qs = q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32)
    if fmt == "fp8":
        cache_dev = L.index_cache[0]
        ref = orc.indexer_logits(q8, qs, wt, w.row_req, pos, w.page_table, oracle_index_cache(w), stride)
        logits_fn, topk_fn = dsa.dsa_indexer_logits, dsa.dsa_indexer_topk
    else:
        cache_dev = L.build_mxfp4_index(0)
        treq, tpos = all_tokens(w)
        mx = np.zeros((w.num_pages, 4352), np.uint8)
        orc.index_k_store_mxfp4(raw_k(w), treq, tpos, w.page_table, mx)
        ref = orc.indexer_logits_mxfp4(q8, qs, wt, w.row_req, pos, w.page_table, mx, stride)
        logits_fn, topk_fn = dsa.dsa_indexer_logits_mxfp4, dsa.dsa_indexer_topk_mxfp4
    for r in pad:
        assert np.all(np.isneginf(ref[r])), "the oracle's padded row is all -inf"
    logits = torch.full((w.R, stride), float("nan"), dtype=torch.float32, device=DEV)
    logits_fn(L.q8, L.qs, L.w_head, rows, L.pages, cache_dev, logits)
    torch.cuda.synchronize()
    got = host(logits)
    for r in pad:
        assert np.all(np.isneginf(got[r])), f"padded row {r}: not all -inf ({np.isnan(got[r]).sum()} unwritten)"
    assert_logits_close(got, ref)
    # the separate top-k and the fused indexer + top-k: padded rows select nothing
    ridx, kth = orc.topk(ref, pos, 2048)
    ws = torch.empty(max(dsa.dsa_topk_workspace_size(w.R, stride, 2048), 256), dtype=torch.uint8, device=DEV)
    idx = torch.full((w.R, 2048), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(logits, rows, 2048, idx, ws)
    torch.cuda.synchronize()
    sep = host(idx)
    for r in pad:
        assert np.all(sep[r] == -1), f"padded row {r} selected positions"
    topk_sets_match(sep, ridx, ref, kth)                  # differences only at near-ties
    idx.fill_(-7)
    logits.fill_(float("nan"))
    with topk_path(path):
        topk_fn(L.q8, L.qs, L.w_head, rows, L.pages, cache_dev, logits, 2048, idx, ws)
    torch.cuda.synchronize()
    fused = host(idx)
    for r in pad:
        assert np.all(fused[r] == -1), f"padded row {r} selected positions"
    assert np.array_equal(fused, sep)                     # same scores, same exact selection
    dsa.dsa_check_device_errors()


def _mla_case(w, pad, k, seed):
    cache = oracle_latent_cache(w, 0)
    _, _, qm = queries(w, [0])
    pos = _padded(w, pad)
    rng = np.random.default_rng(seed)
    idx = np.full((w.R, k), -1, np.int32)
    for r in range(w.R):
        p = int(w.row_pos[r])               # padded rows get real-looking indices: ignored
        sel = rng.choice(p + 1, size=min(k, p + 1), replace=False)
        idx[r, :len(sel)] = sel
    ref, rlse = orc.sparse_mla(qm[0], w.row_req, pos, w.page_table, cache, idx, SM)
    return cache, qm, pos, idx, ref, rlse


def _check_mla(w, pad, out, lse, ref, rlse):
    g, gl = host(out), host(lse)
    for r in pad:
        assert not g[r].any(), f"padded row {r}: output not zero"
        assert np.all(np.isneginf(gl[r])), f"padded row {r}: lse not -inf"
    assert_attention_close(g, ref)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(gl), fin) and np.allclose(gl[fin], rlse[fin], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("fn", ["decode", "prefill"])
def test_mla_padded_rows_split_path(fn):
    """Fewer than 256 rows: split kernels + combine; padded rows in a 6-row group."""
    _announce(f"padded rows: sparse MLA split path ({fn})")
    w = gi.config(2, "small")
    pad = [0, 7, 8, 9, 10, 11, 12, 17]
    cache, qm, pos, idx, ref, rlse = _mla_case(w, pad, 2048, 81)
    out = torch.full((w.R, 64, 512), 0x7FC0, dtype=torch.int16, device=DEV)
    lse = torch.full((w.R, 64), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(dsa.dsa_sparse_mla_workspace_size(w.R, 2048), 256), dtype=torch.uint8, device=DEV)
    f = dsa.dsa_sparse_mla_decode if fn == "decode" else dsa.dsa_sparse_mla_prefill
    f(dev(qm[0].view(np.int16)), _rows(w, pos), dsa.Pages(dev(w.page_table), w.num_pages), dev(cache), dev(idx), out,
      lse, ws)
    torch.cuda.synchronize()
    _check_mla(w, pad, out, lse, ref, rlse)
    dsa.dsa_check_device_errors()


def _stream_workload():
    w = gi.make_decode("mla_stream_pad", gi.SEED_BASE + 82, [2600 + 11 * b for b in range(43)], rows_per_req=6)
    assert w.R == 258
    return w


# rows cut between work-groups sit near every 256th of the tile range; padding covers the first
# row, a whole group, rows next to cuts and the last row
STREAM_PAD = [0, 1, 60, 61, 62, 63, 64, 65, 127, 128, 129, 200, 257]


@pytest.mark.parametrize("k", [2048, 500])
def test_mla_padded_rows_stream_path(k):
    """256 rows or more: the stream-K schedule, with padded rows on both sides of cut rows."""
    _announce(f"padded rows: sparse MLA stream-K path, k={k}")
    w = _stream_workload()
    cache, qm, pos, idx, ref, rlse = _mla_case(w, STREAM_PAD, k, 82 + k)
    out = torch.full((w.R, 64, 512), 0x7FC0, dtype=torch.int16, device=DEV)
    lse = torch.full((w.R, 64), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.zeros(max(dsa.dsa_sparse_mla_workspace_size(w.R, k), 256), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_decode(dev(qm[0].view(np.int16)), _rows(w, pos), dsa.Pages(dev(w.page_table), w.num_pages),
                              dev(cache), dev(idx), out, lse, ws)
    torch.cuda.synchronize()
    _check_mla(w, STREAM_PAD, out, lse, ref, rlse)
    dsa.dsa_check_device_errors()


def test_mla_stream_workspace_stale_reused_and_graph_replayed():
    """One workspace, pre-filled with stale small integers (as a recycled int64 tensor would be),
    used by three eager calls and by a captured graph replayed three times with other work in
    between; every call's output and lse against the oracle."""
    _announce("sparse MLA stream-K: stale workspace, reuse, graph replay")
    w = _stream_workload()
    k = 2048
    cache, qm, pos, idx, ref, rlse = _mla_case(w, [], k, 83)
    nbytes = dsa.dsa_sparse_mla_workspace_size(w.R, k)
    ws = torch.empty((nbytes + 7) // 8, dtype=torch.int64, device=DEV)
    ws.copy_(torch.arange(ws.numel(), dtype=torch.int64, device=DEV) % 5000)    # 0, 1, 2, ... again and again
    q_d, idx_d, cache_d = dev(qm[0].view(np.int16)), dev(idx), dev(cache)
    rows, pages = _rows(w, pos), dsa.Pages(dev(w.page_table), w.num_pages)
    out = torch.empty((w.R, 64, 512), dtype=torch.int16, device=DEV)
    lse = torch.empty((w.R, 64), dtype=torch.float32, device=DEV)
    wsb = ws.view(torch.uint8)

    def call():
        dsa.dsa_sparse_mla_decode(q_d, rows, pages, cache_d, idx_d, out, lse, wsb)

    for i in range(3):
        out.fill_(0x7FC0)
        lse.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        _check_mla(w, [], out, lse, ref, rlse)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(3):
        out.fill_(0x7FC0)
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        _check_mla(w, [], out, lse, ref, rlse)
        x = torch.randn(1 << 20, device=DEV)          # other work between replays
        assert torch.isfinite(x.sum())
    del graph
    dsa.dsa_check_device_errors()
