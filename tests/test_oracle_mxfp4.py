"""Pins for the oracle's MXFP4 index-K variant: the e2m1 element codec (the OCP MX value
table, brute force, ties), the 6-max ue8m0 scale (closed-form boundaries), the 4352-B page
layout written by the store, and MXFP4 indexer logits (NumPy brute force, invariants).

The page ("GLM-5.3 推理全链路(十一)", section on the two non-cache byte streams of the read
path) fixes 128/2 + 128/32 = 68 B per token; the element format is the OCP MX e2m1 one."""
import numpy as np

import dsa_inputs as gi

# The eight e2m1 magnitudes of the OCP MX specification (codes 0..7; 8..15 are their negatives).
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _np_encode(x):
    """Nearest e2m1 code by search over the literal table, ties to the even code, saturating."""
    a = np.minimum(np.abs(x), 6.0)
    d = np.abs(a[:, None] - E2M1[None, :])
    best = np.zeros(len(a), np.int64)
    bd = np.full(len(a), np.inf)
    for c in range(8):
        better = (d[:, c] < bd) | ((d[:, c] == bd) & (c % 2 == 0))
        best = np.where(better, c, best)
        bd = np.where(better, d[:, c], bd)
    return (best | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def test_fp4_decode_is_the_mx_table(orc):
    d = orc.fp4_decode(np.arange(16, dtype=np.uint8))
    assert np.array_equal(d[:8], E2M1)
    assert np.array_equal(d[8:], -E2M1) and np.signbit(d[8])


def test_fp4_roundtrip_and_bruteforce(orc):
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(orc.fp4_encode(orc.fp4_decode(codes)), codes)
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    rng = np.random.default_rng(40)
    rnd = rng.standard_normal(100_000) * 3
    x = np.concatenate([mids, mids * (1 + 1e-12), mids * (1 - 1e-12), -mids, rnd,
                        [0.0, -0.0, 5.999, 6.0, 6.5, 100.0, -100.0]])
    ref = _np_encode(x)
    assert np.array_equal(orc.fp4_encode(x), ref)
    assert np.array_equal(orc.fp4_encode(x, brute=True), ref)


def test_fp4_ties_to_even_code(orc):
    mids = (E2M1[:-1] + E2M1[1:]) / 2          # 0.25 0.75 1.25 1.75 2.5 3.5 5
    assert list(orc.fp4_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]


def test_ue8m0_fp4_boundaries(orc):
    k = np.arange(-20, 20)
    exact = 6.0 * 2.0 ** k
    assert np.array_equal(orc.ue8m0_fp4(exact), 2.0 ** k)
    assert np.array_equal(orc.ue8m0_fp4(exact * (1 + 2.0 ** -40)), 2.0 ** (k + 1))
    assert np.array_equal(orc.ue8m0_fp4(exact * (1 - 2.0 ** -40)), 2.0 ** k)
    assert orc.ue8m0_fp4(np.array([0.0]))[0] == 1.0
    rng = np.random.default_rng(41)
    a = rng.random(10000) * 2.0 ** rng.integers(-30, 30, 10000) + 1e-30
    s = orc.ue8m0_fp4(a)
    assert np.all(a <= 6.0 * s) and np.all(a > 3.0 * s)


def _unpack_key(page, slot):
    """Key `slot` of an MXFP4 page -> 128 dequantised dims, from the layout alone."""
    codes = page[slot * 64:(slot + 1) * 64]
    nib = np.empty(128, np.uint8)
    nib[0::2] = codes & 0xF
    nib[1::2] = codes >> 4
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sb = page[4096 + 4 * slot:4096 + 4 * slot + 4].astype(np.int64)
    return mag * np.repeat(2.0 ** (sb - 127), 32), nib, sb


def test_store_layout_and_quantisation(orc):
    n = 150
    rng = np.random.default_rng(42)
    k = orc.bf16_from_double(rng.standard_normal((n, 128)))
    pos = np.arange(n, dtype=np.int32) * 7 % 300
    pos[5] = -1                                        # padded token: nothing written
    pt = gi.permutation(42, 9, 5).astype(np.int32)[None, :]
    cache = np.full((5, 64 * 68), 0xAB, np.uint8)
    orc.index_k_store_mxfp4(k, np.zeros(n, np.int32), pos, pt, cache)
    y = orc.ln_rope(orc.bf16_to_double(k), pos.astype(np.int64))
    for t in range(n):
        p = int(pos[t])
        if p < 0:
            continue
        page = cache[pt[0, p // 64]]
        val, nib, sb = _unpack_key(page, p % 64)
        for b in range(4):
            blk = y[t, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            e = int(np.log2(orc.ue8m0_fp4(np.array([amax]))[0]))
            assert sb[b] == e + 127
            assert np.array_equal(nib[32 * b:32 * b + 32], _np_encode(blk / 2.0 ** e))
    # the padded token would have sat at position 35 (no other token does): never written
    assert 35 not in pos
    page0 = cache[pt[0, 0]]
    assert np.all(page0[35 * 64:36 * 64] == 0xAB) and np.all(page0[4096 + 4 * 35:4096 + 4 * 36] == 0xAB)


def test_store_error_bound(orc):
    """Dequantised key within half an e2m1 step (times the block scale) of LN + RoPE."""
    n = 64
    rng = np.random.default_rng(43)
    k = orc.bf16_from_double(rng.standard_normal((n, 128)) * 3 + 1)
    pos = np.arange(n, dtype=np.int32)
    pt = np.array([[0]], np.int32)
    cache = np.zeros((1, 64 * 68), np.uint8)
    orc.index_k_store_mxfp4(k, np.zeros(n, np.int32), pos, pt, cache)
    y = orc.ln_rope(orc.bf16_to_double(k), pos.astype(np.int64))
    gap = np.array([0.25, 0.25, 0.25, 0.25, 0.5, 0.5, 1.0, 1.0])      # half the step above each magnitude
    for t in range(n):
        val, nib, sb = _unpack_key(cache[0], t)
        sc = np.repeat(2.0 ** (sb.astype(np.int64) - 127), 32)
        assert np.all(np.abs(val - y[t]) <= gap[nib & 7] * sc + 1e-15)


def _mx_setup(n_tok=300, R=3, seed=44):
    pt = gi.permutation(seed, 9, (n_tok + 63) // 64).astype(np.int32)[None, :]
    rng = np.random.default_rng(seed)
    cache = rng.integers(0, 256, (pt.shape[1], 64 * 68)).astype(np.uint8)
    cache[:, 4096:] = rng.integers(120, 131, (pt.shape[1], 256))      # scales 2^-7 .. 2^3
    q8 = (rng.integers(0, 256, (R, 32, 128)) & 0xF7).astype(np.uint8)
    qs = (2.0 ** rng.integers(-6, 2, (R, 32))).astype(np.float32)
    w = rng.random((R, 32)).astype(np.float32)
    pos = np.array([n_tok - 1, n_tok // 2, 5][:R], np.int32)
    return pt, cache, q8, qs, w, pos


def test_logits_mxfp4_bruteforce(orc):
    pt, cache, q8, qs, w, pos = _mx_setup()
    lg = orc.indexer_logits_mxfp4(q8, qs, w, np.zeros(3, np.int32), pos, pt, cache)
    q = orc.fp8_decode(q8) * qs[:, :, None]
    for r in range(3):
        for s in range(lg.shape[1]):
            if s > pos[r]:
                assert np.isneginf(lg[r, s])
                continue
            key, _, _ = _unpack_key(cache[pt[0, s // 64]], s % 64)
            ref = np.sum(w[r].astype(np.float64) * np.maximum(q[r] @ key, 0))
            assert lg[r, s] == np.float32(ref) or abs(lg[r, s] - ref) <= 1e-6 * abs(ref)


def test_logits_mxfp4_invariants(orc):
    pt, cache, q8, qs, w, pos = _mx_setup()
    req = np.zeros(3, np.int32)
    lg = orc.indexer_logits_mxfp4(q8, qs, w, req, pos, pt, cache)
    fin = np.isfinite(lg)
    assert np.all(lg[fin] >= 0)
    # a key block's scale one step up doubles that block's contribution: with every block
    # scaled, the whole score doubles exactly
    c2 = cache.copy()
    c2[:, 4096:] += 1
    lg2 = orc.indexer_logits_mxfp4(q8, qs, w, req, pos, pt, c2)
    assert np.array_equal(lg2[fin], lg[fin] * 2)
    perm = np.random.default_rng(1).permutation(cache.shape[0])
    c3 = np.empty_like(cache)
    c3[perm] = cache
    assert np.array_equal(orc.indexer_logits_mxfp4(q8, qs, w, req, pos, perm[pt].astype(np.int32), c3), lg)


def test_mxfp4_bytes_per_token(orc):
    # 128/2 B of codes + 128/32 scale bytes = 68 B, about half of FP8's 132
    assert orc.IDX_MXFP4_PAGE_BYTES == 64 * (128 // 2 + 128 // 32) == 4352


def test_mxfp4_topk_overlap_with_fp8(orc):
    """Measurement, not a pin: the share of the FP8 cache's top-2048 that the MXFP4 cache keeps
    on the decode-batch inputs (the page leaves the effect of the coarser keys on the top-k
    open).  A loose floor only guards against a broken variant."""
    from parity import LN_EPS, THETA, all_tokens, oracle_index_cache, queries, raw_k
    w = gi.config(1, "small")
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    q8, qs = q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32)
    req, pos = all_tokens(w)
    mx = np.zeros((w.num_pages, 64 * 68), np.uint8)
    orc.index_k_store_mxfp4(raw_k(w), req, pos, w.page_table, mx, LN_EPS, THETA)
    lg8 = orc.indexer_logits(q8, qs, wt, w.row_req, w.row_pos, w.page_table, oracle_index_cache(w))
    lg4 = orc.indexer_logits_mxfp4(q8, qs, wt, w.row_req, w.row_pos, w.page_table, mx)
    i8, _ = orc.topk(lg8, w.row_pos, 2048)
    i4, _ = orc.topk(lg4, w.row_pos, 2048)
    ov = [len(set(a[a >= 0]) & set(b[b >= 0])) / max(1, int((a >= 0).sum())) for a, b in zip(i8, i4)]
    print(f"MXFP4 keeps {np.mean(ov):.3f} of the FP8 top-2048 on average (min {np.min(ov):.3f})")
    assert np.mean(ov) > 0.5
