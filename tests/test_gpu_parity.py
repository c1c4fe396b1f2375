"""GPU parity: every libdsa entry point against the CPU oracle on identical seeded inputs.

Stage tests feed each kernel inputs built by the oracle (uploaded), so a stage is judged
alone; layer tests run the whole path on the GPU (stores included) and compare every
intermediate with the oracle's own pipeline on the same seeds.
"""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import (LN_EPS, SM, THETA, assert_attention_close, assert_logits_close, bf16_to_f64, needle_overrides,
                    oracle_index_cache, oracle_latent_cache, queries, topk_path, topk_sets_match)

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


def rows_of(w):
    return dsa.Rows(dev(w.row_req), dev(w.row_pos), w.max_pos, w.rows_per_req)


def pages_of(w):
    return dsa.Pages(dev(w.page_table), w.num_pages)


def _announce(name):
    print(f"\n[gpu] {name}", flush=True)


# ----------------------------------------------------------------------------- stages
def test_quant_fp8_bit_exact():
    _announce("quant_fp8")
    x = gi.normal_bf16(3, 1, 0, 4096 * 128).reshape(4096, 128)
    x[0] = 0                                                  # all-zero block -> scale 1
    x[1] = orc.bf16_from_double(np.linspace(-1e-30, 1e-30, 128))   # tiny (subnormal-range) values
    x[2] = orc.bf16_from_double(np.linspace(-3e38, 3e38, 128))     # near the bf16 maximum
    x[3] = orc.bf16_from_double(448.0 * 2.0 ** np.arange(-64, 64))  # exact scale boundaries
    codes, scale = orc.quant_fp8(x)
    y = torch.empty((4096, 128), dtype=torch.uint8, device=DEV)
    s = torch.empty(4096, dtype=torch.float32, device=DEV)
    dsa.dsa_quant_fp8(dev(x.view(np.int16)), y, s)
    torch.cuda.synchronize()
    assert np.array_equal(host(s), scale)
    assert np.array_equal(host(y), codes)


@pytest.mark.parametrize("cid", [0, 1, 2])
def test_stores_bit_exact(cid):
    _announce(f"stores c{cid}")
    w = gi.config(cid, "small")
    L = DeviceLayer(w)
    torch.cuda.synchronize()
    ref = oracle_index_cache(w)
    got = host(L.index_cache[0])
    diff = np.argwhere(got != ref)
    assert len(diff) == 0, f"{len(diff)} index-K bytes differ, first at {diff[:5].tolist()}"
    for l in L.layers:
        assert np.array_equal(host(L.latent_cache[l]), oracle_latent_cache(w, l)), f"latent layer {l}"
    dsa.dsa_check_device_errors()


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_logits_stage(cid):
    _announce(f"logits c{cid}")
    w = gi.config(cid, "small")
    cache = oracle_index_cache(w)
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    q8, qs = q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32)
    ref = orc.indexer_logits(q8, qs, wt, w.row_req, w.row_pos, w.page_table, cache)
    logits = torch.full(ref.shape, float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_logits(dev(q8), dev(qs), dev(wt), rows_of(w), pages_of(w), dev(cache), logits)
    torch.cuda.synchronize()
    assert_logits_close(host(logits), ref)


def _topk_gpu(logits, pos, k=2048, group=1):
    R, stride = logits.shape
    rows = dsa.Rows(dev(np.zeros(R, np.int32)), dev(pos), int(pos.max()), group)
    ws = torch.empty(dsa.dsa_topk_workspace_size(R, stride, k), dtype=torch.uint8, device=DEV)
    idx = torch.full((R, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(dev(logits), rows, k, idx, ws)
    torch.cuda.synchronize()
    return host(idx)


def test_topk_stage_exact():
    _announce("topk stage")
    rng = np.random.default_rng(5)
    R, n = 9, 40000
    stride = orc.logits_stride(n - 1)
    lg = np.full((R, stride), -np.inf, np.float32)
    lg[:, :n] = np.abs(rng.standard_normal((R, n))).astype(np.float32) * 10
    lg[1, :n] = np.round(lg[1, :n] * 4) / 4                # heavy exact ties around the threshold
    lg[2, :n] = 1.0                                       # all equal: lowest positions win
    lg[3, :n] = rng.integers(0, 3, n).astype(np.float32)  # > 4096 candidates in the threshold bin
    pos = np.array([n - 1, n - 1, n - 1, n - 1, 2047, 2048, 100, -1, 30000], np.int32)
    ref, kth = orc.topk(lg, pos, 2048)
    got = _topk_gpu(lg, pos)
    assert np.array_equal(got, ref)
    # small k as well
    ref8, _ = orc.topk(lg, pos, 8)
    assert np.array_equal(_topk_gpu(lg, pos, 8), ref8)


@pytest.mark.parametrize("n", [2049, 8192, 8193, 32768, 32769])
def test_topk_stage_exact_at_kernel_limits(n):
    """The patterns above at row lengths on both sides of the one-work-group top-k's limits
    (8,192 scores for its 256-thread form, 32,768 for 1024 threads; a call whose longest row is
    longer takes the multi-kernel radix), for k = 2048, 1000 and 8."""
    _announce(f"topk stage at n={n}")
    rng = np.random.default_rng(n)
    stride = orc.logits_stride(n - 1)
    lg = np.full((8, stride), -np.inf, np.float32)
    lg[:, :n] = np.abs(rng.standard_normal((8, n))).astype(np.float32) * 10
    lg[1, :n] = np.round(lg[1, :n] * 4) / 4                # heavy exact ties around the threshold
    lg[2, :n] = 1.0                                       # all equal: lowest positions win
    lg[3, :n] = rng.integers(0, 3, n).astype(np.float32)  # far more ties than the work-group has threads
    pos = np.array([n - 1, n - 1, n - 1, n - 1, 2047, 2048, -1, n // 2], np.int32)
    for k in (2048, 1000, 8):
        ref, _ = orc.topk(lg, pos, k)
        assert np.array_equal(_topk_gpu(lg, pos, k), ref), f"k={k}"


@pytest.mark.parametrize("n", [40000, 1048576])
def test_topk_output_order_bucket_patterns(n):
    """Rows longer than the one-work-group top-k: the multi-kernel radix writes the selection
    ascending by a counting sort on the positions' high bits (2048 buckets).  Selections that fill
    a few buckets completely (a contiguous block at the start, in the middle, at the end), one
    position per bucket, and a random spread, against the oracle, for k = 2048 and 100."""
    _announce(f"topk output order, bucket patterns, n={n}")
    rng = np.random.default_rng(n + 11)
    stride = orc.logits_stride(n - 1)
    R = 5
    lg = np.full((R, stride), -np.inf, np.float32)
    lg[:, :n] = rng.random((R, n), dtype=np.float32)
    hi = 2.0 + rng.random(2048, dtype=np.float32)          # planted scores above every other
    lg[0, :2048] = hi                                      # block at the start
    mid = (n // 2) & ~511
    lg[1, mid:mid + 2048] = hi                             # block in the middle, bucket-aligned
    lg[2, n - 2048:n] = hi                                 # block at the end
    step = n // 2048
    lg[3, np.arange(2048) * step] = hi                     # one position per bucket
    pos = np.full(R, n - 1, np.int32)                      # row 4: the random spread
    for k in (2048, 100):
        ref, _ = orc.topk(lg, pos, k)
        got = _topk_gpu(lg, pos, k)
        assert np.array_equal(got, ref), f"k={k}"
        assert (np.diff(got, axis=1) > 0).all(), "ascending"


@pytest.mark.parametrize("cid", [0, 2])
def test_mla_stage(cid):
    _announce(f"mla stage c{cid}")
    w = gi.config(cid, "small")
    cache = oracle_latent_cache(w, 0)
    _, _, qm = queries(w, [0])
    rng = np.random.default_rng(cid)
    idx = np.full((w.R, 2048), -1, np.int32)
    for r in range(w.R):
        p = int(w.row_pos[r])
        sel = rng.choice(p + 1, size=min(2048, p + 1), replace=False)
        idx[r, :len(sel)] = sel
    idx[0, 5] = int(w.row_pos[0]) + 1 if w.row_pos[0] + 1 < w.ctx[0] else -1   # beyond the row: masked
    idx[0, 6] = idx[0, 7]                                                     # a repeated position
    ref, rlse = orc.sparse_mla(qm[0], w.row_req, w.row_pos, w.page_table, cache, idx, SM)
    out = torch.empty((w.R, 64, 512), dtype=torch.int16, device=DEV)
    lse = torch.empty((w.R, 64), dtype=torch.float32, device=DEV)
    nm = dsa.dsa_sparse_mla_workspace_size(w.R, 2048)
    ws = torch.empty(max(nm, 256), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_decode(dev(qm[0].view(np.int16)), rows_of(w), pages_of(w), dev(cache), dev(idx), out, lse, ws)
    torch.cuda.synchronize()
    err = assert_attention_close(host(out), ref)
    assert np.allclose(host(lse), rlse, rtol=1e-4, atol=1e-4)
    print(f"  max abs err {err:.3g}")


@pytest.mark.parametrize("k", [512, 500])
def test_mla_stream_schedule_many_rows(k):
    """R >= 256 rows take the stream-K schedule (rows cut across work-groups and merged by the
    second writer); every row is checked, with a ragged last tile when k % 32 != 0."""
    _announce(f"mla stream schedule R=258 k={k}")
    w = gi.make_decode("mla_stream", gi.SEED_BASE + 60, [3000 + 7 * b for b in range(43)], rows_per_req=6)
    assert w.R == 258
    cache = oracle_latent_cache(w, 0)
    _, _, qm = queries(w, [0])
    rng = np.random.default_rng(k)
    idx = np.full((w.R, k), -1, np.int32)
    for r in range(w.R):
        p = int(w.row_pos[r])
        sel = rng.choice(p + 1, size=min(k, p + 1), replace=False)
        idx[r, :len(sel)] = sel
    idx[3, 100:] = -1                                   # a row with few valid keys
    idx[7, :] = -1                                      # a row with none
    ref, rlse = orc.sparse_mla(qm[0], w.row_req, w.row_pos, w.page_table, cache, idx, SM)
    out = torch.empty((w.R, 64, 512), dtype=torch.int16, device=DEV)
    lse = torch.empty((w.R, 64), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(dsa.dsa_sparse_mla_workspace_size(w.R, k), 256), dtype=torch.uint8, device=DEV)
    for _ in range(2):                                  # the slot counters are reset on every call
        out.fill_(0x7FC0)
        dsa.dsa_sparse_mla_decode(dev(qm[0].view(np.int16)), rows_of(w), pages_of(w), dev(cache), dev(idx), out, lse, ws)
        torch.cuda.synchronize()
        assert_attention_close(host(out), ref)
        g = host(lse)
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(g), fin) and np.allclose(g[fin], rlse[fin], rtol=1e-4, atol=1e-4)
    dsa.dsa_check_device_errors()


def test_mla_special_cases():
    _announce("mla special cases")
    w = gi.config(0, "small")
    cache = oracle_latent_cache(w, 0)
    _, _, qm = queries(w, [0])
    idx = np.full((1, 2048), -1, np.int32)
    idx[0, 100] = 777                                     # one valid index -> exact copy of its latent
    ref, _ = orc.sparse_mla(qm[0], w.row_req, w.row_pos, w.page_table, cache, idx, SM)
    out = torch.empty((1, 64, 512), dtype=torch.int16, device=DEV)
    lse = torch.empty((1, 64), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(dsa.dsa_sparse_mla_workspace_size(1, 2048), 256), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_decode(dev(qm[0].view(np.int16)), rows_of(w), pages_of(w), dev(cache), dev(idx), out, lse, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint16), ref)
    idx[:] = -1                                           # nothing selected -> zeros, lse = -inf
    dsa.dsa_sparse_mla_decode(dev(qm[0].view(np.int16)), rows_of(w), pages_of(w), dev(cache), dev(idx), out, lse, ws)
    torch.cuda.synchronize()
    assert not host(out).any() and np.all(np.isneginf(host(lse)))


# ----------------------------------------------------------------------------- whole layer
@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_layer_end_to_end(cid):
    _announce(f"layer end-to-end c{cid}")
    w = gi.config(cid, "small")
    ov = needle_overrides(w) if w.needles is not None else None
    L = DeviceLayer(w, k_overrides=ov)
    L.group_step()
    torch.cuda.synchronize()
    # oracle pipeline on the same seeds
    cache = oracle_index_cache(w, ov)
    assert np.array_equal(host(L.index_cache[0]), cache)
    q, wt, qm = queries(w, L.layers)
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    assert np.array_equal(host(L.q8).reshape(-1, 128), q8) and np.array_equal(host(L.qs).reshape(-1), qs)
    q8, qs = q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32)
    lg = orc.indexer_logits(q8, qs, wt, w.row_req, w.row_pos, w.page_table, cache)
    # the fused indexer + top-k keeps its logits buffer as scratch: score separately to check them
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    torch.cuda.synchronize()
    assert_logits_close(host(L.logits), lg)
    ridx, kth = orc.topk(lg, w.row_pos, 2048)
    gidx = host(L.idx)
    ndiff = topk_sets_match(gidx, ridx, lg, kth)
    if w.needles is not None:
        assert set(gidx[0].tolist()) == set(w.needles.tolist()), "top-k must be exactly the needle set"
    same = [r for r in range(w.R) if set(gidx[r]) == set(ridx[r])]
    assert len(same) >= w.R - max(1, w.R // 50), f"{ndiff} rows differ at near-ties"
    for l in L.layers:                                   # layer 0 full, others shared (same idx tensor)
        lat = oracle_latent_cache(w, l)
        ref, _ = orc.sparse_mla(qm[l], w.row_req, w.row_pos, w.page_table, lat, ridx, SM)
        assert_attention_close(host(L.out[l])[same], ref[same])
    dsa.dsa_check_device_errors()


def test_shared_layers_reuse_the_same_index_tensor():
    _announce("shared layer reuse")
    w = gi.config(2, "small")
    L = DeviceLayer(w)
    seen = []
    orig = dsa.dsa_sparse_mla_decode

    def spy(q, rows, pages, latent, idx, *a, **k):
        seen.append(idx.data_ptr())
        return orig(q, rows, pages, latent, idx, *a, **k)

    dsa.dsa_sparse_mla_decode = spy
    try:
        L.group_step()
    finally:
        dsa.dsa_sparse_mla_decode = orig
    torch.cuda.synchronize()
    assert len(seen) == 4 and len(set(seen)) == 1 and seen[0] == L.idx.data_ptr()
    # the group is GLM-5.3 layers 6..9: one full layer followed by three shared ones
    assert [dsa.dsa_layer_is_shared(l, topk_freq=4, skip_topk_offset=3) for l in range(6, 10)] == [False, True, True, True]


def test_determinism_and_page_permutation():
    _announce("determinism / page permutation")
    w = gi.config(1, "small")
    A = DeviceLayer(w)
    A.group_step()
    first = (host(A.idx).copy(), host(A.out[0]).copy())
    A.group_step()
    assert np.array_equal(host(A.idx), first[0])
    assert np.array_equal(host(A.out[0]), first[1])
    # same logical content under a different page permutation
    w2 = gi.config(1, "small")
    perm = np.random.default_rng(1).permutation(w2.num_pages).astype(np.int32)
    w2.page_table = perm[w2.page_table]
    B = DeviceLayer(w2)
    B.group_step()
    torch.cuda.synchronize()
    assert np.array_equal(host(B.idx), first[0])
    assert np.array_equal(host(B.out[0]), first[1])


def test_bad_page_id_is_flagged_not_dereferenced():
    _announce("bad page id")
    w = gi.config(0, "small")
    cache = torch.zeros((w.num_pages, 8448), dtype=torch.uint8, device=DEV)
    pt = w.page_table.copy()
    pt[0, 3] = w.num_pages + 1000                          # out of the pool: must be skipped
    k = torch.zeros((w.total_tokens, 128), dtype=torch.int16, device=DEV)
    rows = dsa.Rows(dev(np.zeros(w.total_tokens, np.int32)), dev(np.arange(w.total_tokens, dtype=np.int32)),
                    w.total_tokens - 1)
    dsa.dsa_index_k_store(k, rows, dsa.Pages(dev(pt), w.num_pages), cache)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_check_device_errors()
    assert e.value.status == 5
    dsa.dsa_check_device_errors()                          # the flag was cleared


@pytest.mark.parametrize("path", ["direct", "filtered"])
@pytest.mark.parametrize("cid", [1, 2, 3])
def test_fused_indexer_topk_equals_separate_calls(cid, path):
    _announce(f"fused indexer+topk c{cid}, {path} path")
    w = gi.config(cid, "small")
    L = DeviceLayer(w)
    dsa.dsa_quant_fp8(L.q_idx, L.q8, L.qs)
    with topk_path(path):
        L.indexer_topk(0)
    torch.cuda.synchronize()
    fused_idx = host(L.idx).copy()
    dsa.dsa_indexer_logits(L.q8, L.qs, L.w_head, L.rows, L.pages, L.index_cache[0], L.logits)
    dsa.dsa_topk(L.logits, L.rows, 2048, L.idx, L.ws_topk)
    torch.cuda.synchronize()
    assert np.array_equal(host(L.idx), fused_idx)      # same scores, same exact selection
