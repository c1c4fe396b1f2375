"""Pins for indexer logits (NumPy brute force, invariants) and top-k (full sort, short-context
rule, ties, needle closed form)."""
import numpy as np

import dsa_inputs as gi


def _setup(n_tok=300, R=3, seed=21):
    pt = gi.permutation(seed, 9, (n_tok + 63) // 64).astype(np.int32)[None, :]
    rng = np.random.default_rng(seed)
    cache = np.zeros((pt.shape[1], 8448), np.uint8)
    cache[:, :8192] = rng.integers(0, 256, (pt.shape[1], 8192)) & 0xF7   # no NaN codes
    cache[:, 8192:] = np.array(2.0 ** rng.integers(-8, 3, (pt.shape[1], 64)), np.float32).view(np.uint8).reshape(-1, 256)
    q8 = (rng.integers(0, 256, (R, 32, 128)) & 0xF7).astype(np.uint8)
    qs = (2.0 ** rng.integers(-6, 2, (R, 32))).astype(np.float32)
    w = rng.random((R, 32)).astype(np.float32)
    pos = np.array([n_tok - 1, n_tok // 2, 5][:R], np.int32)
    return pt, cache, q8, qs, w, pos


def _brute(orc, pt, cache, q8, qs, w, pos, stride):
    R = q8.shape[0]
    out = np.full((R, stride), -np.inf)
    q = orc.fp8_decode(q8) * qs[:, :, None]
    for r in range(R):
        for s in range(pos[r] + 1):
            pg = cache[pt[0, s // 64]]
            k = orc.fp8_decode(pg[(s % 64) * 128:(s % 64 + 1) * 128]) * pg[8192 + 4 * (s % 64):8196 + 4 * (s % 64)].view(np.float32)[0]
            out[r, s] = np.sum(w[r] * np.maximum(q[r] @ k, 0))
    return out


def test_logits_bruteforce(orc):
    pt, cache, q8, qs, w, pos = _setup()
    lg = orc.indexer_logits(q8, qs, w, np.zeros(3, np.int32), pos, pt, cache)
    assert lg.shape == (3, 512)
    ref = _brute(orc, pt, cache, q8, qs, w, pos, 512)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.allclose(lg[fin], ref[fin], rtol=1e-6, atol=0)


def test_logits_invariants(orc):
    pt, cache, q8, qs, w, pos = _setup()
    req = np.zeros(3, np.int32)
    lg = orc.indexer_logits(q8, qs, w, req, pos, pt, cache)
    assert np.all(lg[np.isfinite(lg)] >= 0)
    # power-of-two scaling of q scales the logits exactly
    lg2 = orc.indexer_logits(q8, qs * 8, w, req, pos, pt, cache)
    assert np.array_equal(lg2[np.isfinite(lg)], lg[np.isfinite(lg)] * 8)
    # moving pages (same logical content) changes nothing
    perm = np.random.default_rng(0).permutation(cache.shape[0])
    cache2 = np.empty_like(cache)
    cache2[perm] = cache
    lg3 = orc.indexer_logits(q8, qs, w, req, pos, perm[pt].astype(np.int32), cache2)
    assert np.array_equal(lg3, lg)
    # a padded row (pos -1) sees nothing
    lg4 = orc.indexer_logits(q8, qs, w, req, np.array([-1, 3, 4], np.int32), pt, cache, stride=256)
    assert np.all(np.isneginf(lg4[0]))


def test_logits_stride_rule(orc):
    assert orc.logits_stride(0) == 256 and orc.logits_stride(255) == 256 and orc.logits_stride(256) == 512
    assert orc.logits_stride(131071) == 131072


def test_topk_full_sort(orc):
    rng = np.random.default_rng(8)
    R, n = 5, 3000
    lg = rng.standard_normal((R, n)).astype(np.float32)
    lg[:, 100:110] = lg[0, 50]                 # a run of exact ties
    pos = np.array([2999, 2500, 2047, 2048, 100], np.int32)
    idx, kth = orc.topk(lg, pos, 2048)
    for r in range(R):
        m = pos[r] + 1
        if m <= 2048:
            assert np.array_equal(idx[r, :m], np.arange(m)) and np.all(idx[r, m:] == -1)
            continue
        order = np.lexsort((np.arange(m), -lg[r, :m]))     # score desc, position asc
        assert np.array_equal(idx[r], np.sort(order[:2048]))
        assert kth[r] == lg[r, order[2047]]


def test_topk_ties_take_lowest_positions(orc):
    lg = np.zeros((1, 5000), np.float32)
    idx, _ = orc.topk(lg, np.array([4999], np.int32), 2048)
    assert np.array_equal(idx[0], np.arange(2048))


def test_topk_padded_and_small(orc):
    lg = np.zeros((2, 256), np.float32)
    idx, _ = orc.topk(lg, np.array([-1, 0], np.int32), 2048)
    assert np.all(idx[0] == -1) and idx[1, 0] == 0 and np.all(idx[1, 1:] == -1)


def test_needle_closed_form(orc):
    """Keys planted along the query's weighted direction are exactly the top-k set."""
    L, k = 6000, 512
    seed = 99
    pt = gi.permutation(seed, 9, (L + 63) // 64).astype(np.int32)[None, :]
    q = gi.normal_bf16(seed, 1, 0, 32 * 128).reshape(1, 32, 128)
    q8, qs = orc.quant_fp8(q.reshape(32, 128))
    w = gi.uniform_f32(seed, 3, 0, 32, gi.w_scale()).reshape(1, 32)
    u = (orc.fp8_decode(q8) * qs[:, None] * w[0][:, None]).sum(0)
    needles = gi.choose_distinct(seed, 11, L - 1, k)
    raw = gi.normal_bf16(seed, 2, 0, L * 128).reshape(L, 128)
    v = orc.ln_rope(np.repeat(u[None], k, 0), needles, ln=False, inverse=True)
    v -= v.mean(1, keepdims=True)
    v *= np.sqrt(128) / np.linalg.norm(v, axis=1, keepdims=True)
    raw[needles] = orc.bf16_from_double(v)
    cache = np.zeros((pt.shape[1], 8448), np.uint8)
    orc.index_k_store(raw, np.zeros(L, np.int32), np.arange(L, dtype=np.int32), pt, cache)
    lg = orc.indexer_logits(q8[None], qs[None], w, np.zeros(1, np.int32), np.array([L - 1], np.int32), pt, cache)
    nd = np.zeros(L, bool)
    nd[needles] = True
    assert lg[0, :L][nd].min() > 1.5 * lg[0, :L][~nd].max()
    idx, _ = orc.topk(lg, np.array([L - 1], np.int32), k)
    assert np.array_equal(idx[0], needles)
