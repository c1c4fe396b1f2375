"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark uses.

The GPU runs the whole layer (group) over every request; the oracle recomputes sampled rows
from the same seeds (only the sampled request's index-K cache and only the selected latent
records are rebuilt on the host).  Also: the short-context path (no scoring when a row sees
at most k positions) and a single-request context sweep from 1K to 128K.
"""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import (SM, assert_attention_close, assert_logits_close, needle_overrides, oracle_index_cache,
                    oracle_index_cache_of, oracle_latent_cache, oracle_latent_cache_of, queries, row_queries,
                    topk_path, topk_sets_match)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402
from sparse_attention_store_amd.workload import DeviceLayer  # noqa: E402


def host(t):
    return t.cpu().numpy()


def take(t, rows):
    """Rows of a device tensor, gathered on the device, as a host array."""
    return host(t[torch.as_tensor(np.asarray(rows), dtype=torch.long, device=t.device)])


def _announce(name):
    print(f"\n[gpu] {name}", flush=True)


def _release(L):
    del L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def check_sampled_rows(w, L, rows, overrides=None, min_same_frac=0.9):
    """Every sampled row: q quantisation bit-exact, logits within tolerance, top-k set equal
    (near-ties excepted), and each layer's attention output against the oracle."""
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    # the fused indexer + top-k keeps the logits buffer as scratch: score separately to check
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    torch.cuda.synchronize()
    n_same = 0
    for b in np.unique(w.row_req[rows]):
        rs = rows[w.row_req[rows] == b]
        cache, pt = oracle_index_cache_of(w, int(b), overrides)
        q, wt, qm = row_queries(w, rs, L.layers)
        q8, qs = orc.quant_fp8(q.reshape(-1, 128))
        assert np.array_equal(take(L.q8, rs).reshape(-1, 128), q8)
        assert np.array_equal(take(L.qs, rs).reshape(-1), qs)
        pos = w.row_pos[rs]
        req0 = np.zeros(len(rs), np.int32)
        lg = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, req0, pos, pt, cache)
        ridx, kth = orc.topk(lg, pos, 2048)
        gidx = take(L.idx, rs)
        long_rows = pos + 1 > 2048              # short rows are not scored by the fused call
        if long_rows.any():
            g_lg = take(L.logits, rs[long_rows])
            ow = lg.shape[1]
            assert_logits_close(g_lg[:, :ow], lg[long_rows])
            assert np.all(np.isneginf(g_lg[:, ow:]))
        topk_sets_match(gidx, ridx, lg, kth)
        same = np.array([set(gidx[i]) == set(ridx[i]) for i in range(len(rs))])
        n_same += int(same.sum())
        for l in L.layers:
            lat, _ = oracle_latent_cache_of(w, int(b), l, ridx)
            ref, rlse = orc.sparse_mla(qm[l], req0, pos, pt, lat, ridx, SM)
            assert_attention_close(take(L.out[l], rs)[same], ref[same])
            assert np.allclose(take(L.lse[l], rs)[same], rlse[same], rtol=1e-4, atol=1e-4)
    assert n_same >= min_same_frac * len(rows), f"only {n_same}/{len(rows)} rows have the oracle's exact set"
    return n_same


def test_full_c1_decode_batch_every_row():
    _announce("full size c1: 32 requests, ctx 8K-32K, every row")
    w = gi.config(1, "full")
    L = DeviceLayer(w)
    L.group_step()
    torch.cuda.synchronize()
    check_sampled_rows(w, L, range(w.R))
    dsa.dsa_check_device_errors()
    _release(L)


def test_full_c2_verify_128k_sampled_requests():
    _announce("full size c2: 64 x 6 rows at 128K, 4-layer group, 8 sampled requests")
    w = gi.config(2, "full")
    L = DeviceLayer(w)
    L.group_step()
    torch.cuda.synchronize()
    reqs = [0, 1, 17, 31, 32, 47, 62, 63]
    rows = [r for r in range(w.R) if int(w.row_req[r]) in reqs]
    check_sampled_rows(w, L, rows)
    dsa.dsa_check_device_errors()
    _release(L)


@pytest.mark.parametrize("path", ["direct", "filtered"])
def test_full_c3_long_1m_needles(path):
    _announce(f"full size c3: 1 request at 1M context, 2048 needles, {path} top-k")
    w = gi.config(3, "full")
    ov = needle_overrides(w)
    L = DeviceLayer(w, k_overrides=ov)
    with topk_path(path):
        L.group_step()
    torch.cuda.synchronize()
    gidx = host(L.idx)[0]
    assert np.array_equal(gidx, np.sort(w.needles)), "top-k must be exactly the needle set, ascending"
    check_sampled_rows(w, L, [0], overrides=ov, min_same_frac=1.0)
    dsa.dsa_check_device_errors()
    _release(L)


def test_full_c4_chunked_prefill_sampled_rows():
    _announce("full size c4: 8192 prefill rows on a 65,536 prefix, 24 sampled rows")
    w = gi.config(4, "full")
    L = DeviceLayer(w)
    L.group_step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    rows = [0, 1, 2, 63, 64, 4095, 8190, 8191] + list(rng.choice(w.R, 16, replace=False))
    check_sampled_rows(w, L, rows)
    dsa.dsa_check_device_errors()
    _release(L)


def test_short_context_rows_skip_scoring():
    """Rows seeing at most k positions take every position and are not scored by the fused
    call (their logits rows stay untouched); the separate logits call still scores them."""
    _announce("short-context path (mixed batch)")
    w = gi.make_decode("short_mix", gi.SEED_BASE + 40, [1000, 2048, 2049, 5000, 64, 1, 2047])
    L = DeviceLayer(w)
    L.logits.fill_(float("nan"))
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    L.indexer_topk(0)
    for l in L.layers:
        L.mla(l)
    torch.cuda.synchronize()
    cache = oracle_index_cache(w)
    q, wt, qm = queries(w, L.layers)
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    lg = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, w.row_req, w.row_pos,
                            w.page_table, cache)
    ridx, kth = orc.topk(lg, w.row_pos, 2048)
    gidx, glg = host(L.idx), host(L.logits)
    short = w.row_pos + 1 <= 2048
    for r in range(w.R):
        if short[r]:
            p = int(w.row_pos[r])
            assert np.array_equal(gidx[r, :p + 1], np.arange(p + 1)) and np.all(gidx[r, p + 1:] == -1)
            assert np.all(np.isnan(glg[r])), f"row {r} (pos {p}) was scored"
    topk_sets_match(gidx, ridx, lg, kth)                 # differences only at near-ties
    same = np.array([set(gidx[r]) == set(ridx[r]) for r in range(w.R)])
    assert same[short].all() and same.sum() >= w.R - 1
    lat = oracle_latent_cache(w, 0)
    ref, _ = orc.sparse_mla(qm[0], w.row_req, w.row_pos, w.page_table, lat, ridx, SM)
    assert_attention_close(host(L.out[0])[same], ref[same])
    # the plain logits call scores every row, short ones included
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    torch.cuda.synchronize()
    assert_logits_close(host(L.logits), lg)
    dsa.dsa_check_device_errors()


def test_short_group_of_six_rows():
    """A request whose six draft rows all sit below k is skipped as a group; the next one is scored."""
    _announce("short-context path (groups of 6)")
    w = gi.make_decode("short_groups", gi.SEED_BASE + 41, [2000, 2051, 3000], rows_per_req=6)
    L = DeviceLayer(w)
    L.logits.fill_(float("nan"))
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    L.indexer_topk(0)
    torch.cuda.synchronize()
    cache = oracle_index_cache(w)
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    lg = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, w.row_req, w.row_pos,
                            w.page_table, cache)
    ridx, kth = orc.topk(lg, w.row_pos, 2048)
    gidx, glg = host(L.idx), host(L.logits)
    assert np.all(np.isnan(glg[:6]))                       # request 0: every row short -> not scored
    topk_sets_match(gidx, ridx, lg, kth)                   # differences only at near-ties
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    torch.cuda.synchronize()
    assert_logits_close(host(L.logits), lg)               # the plain call scores every row
    assert np.array_equal(gidx[:6], ridx[:6])


@pytest.mark.parametrize("ctx", [1024, 2048, 2049, 4096, 16384, 131072])
def test_context_sweep_single_request(ctx):
    _announce(f"context sweep: 1 request, ctx {ctx}")
    w = gi.make_decode(f"sweep_{ctx}", gi.SEED_BASE + 50, [ctx])
    L = DeviceLayer(w)
    L.group_step()
    torch.cuda.synchronize()
    check_sampled_rows(w, L, [0], min_same_frac=1.0)
    dsa.dsa_check_device_errors()
    _release(L)


def filter_pass_chunk(rows_per_group, max_pos, n_groups, fcap=4096, want=2048):
    """Pages per work-group of the fused call's filter pass, as libdsa's launcher picks them: the
    stage of a row group (768 / RG candidates per row up to six rows, 104 for the eight-row
    sub-groups of a long group) bounds the chunk to what a row's share of fcap candidates fits,
    then the chunk halves while fewer than `want` work-groups would run."""
    stage = 768 // rows_per_group if rows_per_group <= 6 else 104
    lim = stage * (max_pos + 1) // (fcap * 64)
    chunk = next((c for c in (128, 64, 32, 16, 8) if lim >= c), 4)
    total_pages = dsa.dsa_logits_stride(max_pos) // 64
    while chunk > 4 and n_groups * -(-total_pages // chunk) < want:
        chunk //= 2
    return chunk


# decode / verify batches whose filter chunks are multiples of 16, and a prefill chunk whose long
# group runs in eight-row sub-groups
REUSE_CASES = [("verify_16x6_128k", [131072] * 16, 6), ("verify_64x6_32k", [32768] * 64, 6),
               ("decode_32x1_128k", [131072 - 5000 * (b % 3) for b in range(32)], 1),
               ("verify_48x3_64k", [65536 - 64 * b for b in range(48)], 3), ("prefill_45000_512", None, 512)]


@pytest.mark.parametrize("name,ctx,rows", REUSE_CASES, ids=[c[0] for c in REUSE_CASES])
def test_fused_equals_separate_where_sampled_pages_are_reused(name, ctx, rows):
    """Filter chunks of 16 pages or more (a multiple of the sampling step): the filter pass takes
    the sampled pages' scores from the sample pass instead of scoring them again.  The selection
    must be exactly that of the separate logits + top-k calls."""
    _announce(f"fused == separate with sampled pages reused: {name}")
    if ctx is None:
        w = gi.make_prefill(name, gi.SEED_BASE + 51, 45000, rows)
        rg, n_groups = 8, rows // 8
    else:
        w = gi.make_decode(name, gi.SEED_BASE + 51, ctx, rows_per_req=rows)
        rg, n_groups = rows, len(ctx)
    chunk = filter_pass_chunk(rg, w.max_pos, n_groups)
    assert chunk >= 16 and chunk % 16 == 0, f"filter chunk {chunk}: the sampled-page reuse would not run"
    L = DeviceLayer(w)
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    with topk_path("filtered"):
        L.indexer_topk(0)
    torch.cuda.synchronize()
    fused = host(L.idx).copy()
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    dsa.dsa_topk(L.logits, L.rows, 2048, L.idx, L.ws_topk)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx), fused)
    dsa.dsa_check_device_errors()
    _release(L)


SAMPLE_STEP = 16    # the fused path scores one page in SAMPLE_STEP to set its filter threshold


def _fused_topk_case(w, overrides, expect_fallback):
    """The filtered path of the fused call on one workload: whether row 0 fell back, its
    selection against the oracle and against the separate calls."""
    L = DeviceLayer(w, k_overrides=overrides)
    L.logits.fill_(float("nan"))
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    with topk_path("filtered"):
        L.indexer_topk(0)
    torch.cuda.synchronize()
    gidx, glg = host(L.idx), host(L.logits)
    # which path the row took: the exact fallback scores every page, the filtered path
    # only the sampled pages and writes no other score
    n = int(w.row_pos[0]) + 1
    unsampled = np.array([s for s in range(n) if (s // 64) % SAMPLE_STEP != 0])
    assert np.isfinite(glg[0, unsampled]).all() == expect_fallback
    cache = oracle_index_cache(w, overrides)
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    lg = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, w.row_req, w.row_pos, w.page_table, cache)
    ridx, kth = orc.topk(lg, w.row_pos, 2048)
    topk_sets_match(gidx, ridx, lg, kth)
    # the unfused path (plain scores + radix top-k) selects the same positions
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    dsa.dsa_topk(L.logits, L.rows, 2048, L.idx, L.ws_topk)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx), gidx)
    # the fused call again, on the workspace the radix top-k just filled (its histograms are
    # not cleared for the filtered path: a flagged row clears its own)
    L.idx.fill_(-7)
    with topk_path("filtered"):
        L.indexer_topk(0)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx), gidx)
    return gidx, ridx


def _too_few_needles(w, n, seed):
    """1000 needles of request 0, 600 of them on sampled pages: the sample sets the threshold
    among the needles, so fewer than k scores pass the filter and the row is flagged."""
    rng = np.random.default_rng(seed)
    sampled = np.array([s for s in range(n - 1) if (s // 64) % SAMPLE_STEP == 0])
    others = np.array([s for s in range(n - 1) if (s // 64) % SAMPLE_STEP != 0])
    return np.sort(np.concatenate([rng.choice(sampled, 600, replace=False), rng.choice(others, 400, replace=False)]))


def _equal_score_key():
    """A raw key whose LayerNorm output is zero on the rotated dims 0..63, so every position
    gets the same stored key and every score of a row is the same number."""
    d = np.arange(1, 33) / 128.0                                  # 1 +- d exact in bf16
    v = np.concatenate([np.ones(64), 1.0 + d, 1.0 - d])          # mean exactly 1
    return orc.bf16_from_double(v)


def test_fused_topk_fallback_when_filter_keeps_too_few():
    _announce("fused top-k: filter keeps fewer than k -> exact fallback")
    n = 30000
    w = gi.make_decode("fb_few", gi.SEED_BASE + 70, [n])
    w.needles = _too_few_needles(w, n, 70)
    gidx, ridx = _fused_topk_case(w, needle_overrides(w), expect_fallback=True)
    assert set(w.needles.tolist()) <= set(gidx[0].tolist())


def test_fused_topk_fallback_long_row_beside_a_filtered_row():
    """A flagged row of 100,000 positions (13 score chunks: each of the fallback's work-groups
    of the row takes several) beside a row of 60,000 that stays on the filtered path."""
    _announce("fused top-k: long flagged row + filtered row")
    n = 100000
    w = gi.make_decode("fb_long", gi.SEED_BASE + 73, [n, 60000])
    w.needles = _too_few_needles(w, n, 73)
    gidx, ridx = _fused_topk_case(w, needle_overrides(w), expect_fallback=True)
    assert set(w.needles.tolist()) <= set(gidx[0].tolist())


def test_fused_topk_fallback_when_candidates_overflow():
    _announce("fused top-k: all scores equal, 9000 candidates -> exact fallback")
    w = gi.make_decode("fb_overflow", gi.SEED_BASE + 71, [9000])
    key = _equal_score_key()
    gidx, ridx = _fused_topk_case(w, {p: key for p in range(9000)}, expect_fallback=True)
    assert np.array_equal(gidx[0], np.arange(2048))       # exact ties keep the lowest positions


def test_fused_topk_ties_inside_candidate_list():
    _announce("fused top-k: all scores equal, 3000 candidates -> exact within the list")
    w = gi.make_decode("fb_ties", gi.SEED_BASE + 72, [3000], rows_per_req=2)
    key = _equal_score_key()
    gidx, ridx = _fused_topk_case(w, {p: key for p in range(3000)}, expect_fallback=False)
    assert np.array_equal(gidx[0], np.arange(2048))


@pytest.mark.parametrize("path", ["direct", "filtered"])
@pytest.mark.parametrize("k", [100, 1000, 2048])
def test_topk_long_rows(k, path):
    """Rows of 300,000 and 600,000 positions (512-position buckets in the output sort; rows of
    over 8,192 samples take the long threshold kernel), for k = 100, 1000 and 2048.  The fused
    and the separate calls against the oracle's set; both ascending and equal."""
    _announce(f"top-k of long rows, k={k}, {path} fused path")
    w = gi.make_decode("long_rows_k", gi.SEED_BASE + 74, [300000, 600000])
    L = DeviceLayer(w, latent_layers=[])
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    cache = oracle_index_cache(w)
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    lg = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, w.row_req, w.row_pos, w.page_table,
                            cache)
    ridx, kth = orc.topk(lg, w.row_pos, k)
    stride = L.logits.shape[-1]
    ws = torch.empty(max(dsa.dsa_topk_workspace_size(w.R, stride, k), 256), dtype=torch.uint8, device="cuda")
    idx = torch.full((w.R, k), -7, dtype=torch.int32, device="cuda")
    with topk_path(path):
        dsa.dsa_indexer_topk(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits, k, idx, ws)
    torch.cuda.synchronize()
    fused = host(idx)
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    idx.fill_(-7)
    dsa.dsa_topk(L.logits, L.rows, k, idx, ws)
    torch.cuda.synchronize()
    sep = host(idx)
    for g in (fused, sep):
        assert np.all(np.diff(g, axis=1) > 0), "positions not strictly ascending"
    assert np.array_equal(fused, sep)
    topk_sets_match(fused, ridx, lg, kth)                 # differences only at near-ties
    dsa.dsa_check_device_errors()


@pytest.mark.parametrize("n", [5000, 30000])
def test_direct_topk_all_equal_scores(n):
    """Every score of the row equal (an empty key range): the one-work-group row top-k of the
    direct path (256 threads up to 8,192 positions, 1024 above) keeps the lowest positions, as
    does the separate top-k over the plain scores."""
    _announce(f"direct-path top-k, {n} equal scores")
    w = gi.make_decode(f"eq_direct_{n}", gi.SEED_BASE + 75, [n])
    key = _equal_score_key()
    L = DeviceLayer(w, latent_layers=[], k_overrides={p: key for p in range(n)})
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    with topk_path("direct"):
        L.indexer_topk(0)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx)[0], np.arange(2048))
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    L.idx.fill_(-7)
    dsa.dsa_topk(L.logits, L.rows, 2048, L.idx, L.ws_topk)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx)[0], np.arange(2048))
    dsa.dsa_check_device_errors()
