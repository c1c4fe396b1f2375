"""Pins for sparse MLA: dense softmax brute force (NumPy), special cases with closed forms."""
import numpy as np

import dsa_inputs as gi


def _setup(n_tok=200, seed=31):
    pt = gi.permutation(seed, 9, (n_tok + 63) // 64).astype(np.int32)[None, :]
    kv = gi.normal_bf16(seed, 5, 0, n_tok * 576).reshape(n_tok, 576)
    return pt, kv


def _store(orc, pt, kv):
    cache = np.zeros((pt.shape[1], 64 * 656), np.uint8)
    n = kv.shape[0]
    orc.latent_store(kv, np.zeros(n, np.int32), np.arange(n, dtype=np.int32), pt, cache)
    return cache


def _deq(orc, pt, cache, s):
    rec = cache[pt[0, s // 64], (s % 64) * 656:(s % 64 + 1) * 656]
    sc = rec[512:528].view(np.float32).astype(np.float64)
    c = orc.fp8_decode(rec[:512]) * np.repeat(sc, 128)
    kr = orc.bf16_to_double(rec[528:].view(np.uint16))
    return np.concatenate([c, kr])


def test_mla_dense_bruteforce(orc):
    pt, kv = _setup()
    cache = _store(orc, pt, kv)
    R = 2
    q = gi.normal_bf16(31, 4, 0, R * 64 * 576).reshape(R, 64, 576)
    idx = np.full((R, 64), -1, np.int32)
    idx[0, :50] = np.arange(0, 200, 4)
    idx[1, :30] = np.arange(30) * 3 + 1
    idx[1, 40] = 190                           # beyond the row position: masked
    pos = np.array([199, 120], np.int32)
    out, lse = orc.sparse_mla(q, np.zeros(R, np.int32), pos, pt, cache, idx)
    qd = orc.bf16_to_double(q)
    for r in range(R):
        sel = [s for s in idx[r] if 0 <= s <= pos[r]]
        K = np.stack([_deq(orc, pt, cache, s) for s in sel])
        lg = qd[r] @ K.T / 16.0
        p = np.exp(lg - lg.max(1, keepdims=True))
        o = (p / p.sum(1, keepdims=True)) @ K[:, :512]
        assert np.array_equal(out[r], orc.bf16_from_double(o))
        assert np.allclose(lse[r], lg.max(1) + np.log(np.exp(lg - lg.max(1, keepdims=True)).sum(1)), rtol=1e-6)


def test_mla_single_index_is_exact_copy(orc):
    pt, kv = _setup()
    cache = _store(orc, pt, kv)
    q = gi.normal_bf16(31, 4, 0, 64 * 576).reshape(1, 64, 576)
    idx = np.full((1, 16), -1, np.int32)
    idx[0, 5] = 77
    out, _ = orc.sparse_mla(q, np.zeros(1, np.int32), np.array([150], np.int32), pt, cache, idx)
    c = _deq(orc, pt, cache, 77)[:512]
    assert np.array_equal(orc.bf16_to_double(out[0]), np.broadcast_to(c, (64, 512)))


def test_mla_zero_query_is_mean(orc):
    pt, kv = _setup()
    cache = _store(orc, pt, kv)
    q = np.zeros((1, 64, 576), np.uint16)
    idx = np.arange(0, 96, dtype=np.int32)[None]
    out, lse = orc.sparse_mla(q, np.zeros(1, np.int32), np.array([199], np.int32), pt, cache, idx)
    mean = np.mean([_deq(orc, pt, cache, s)[:512] for s in range(96)], axis=0)
    assert np.array_equal(out[0, 0], orc.bf16_from_double(mean))
    assert np.allclose(lse, np.log(96))


def test_mla_permutation_duplicates_and_empty(orc):
    pt, kv = _setup()
    cache = _store(orc, pt, kv)
    q = gi.normal_bf16(32, 4, 0, 64 * 576).reshape(1, 64, 576)
    z = np.zeros(1, np.int32)
    p = np.array([199], np.int32)
    idx = np.arange(10, 110, dtype=np.int32)[None]
    a, la = orc.sparse_mla(q, z, p, pt, cache, idx)
    b, lb = orc.sparse_mla(q, z, p, pt, cache, idx[:, ::-1].copy())
    assert np.abs(orc.bf16_to_double(a) - orc.bf16_to_double(b)).max() <= 2.0 ** -8 * np.abs(orc.bf16_to_double(a)).max()
    # a duplicated index counts twice: equal to the softmax with that key's weight doubled
    dup = np.concatenate([idx, [[10]]], 1).astype(np.int32)
    c, _ = orc.sparse_mla(q, z, p, pt, cache, dup)
    K = np.stack([_deq(orc, pt, cache, s) for s in range(10, 110)])
    lg = orc.bf16_to_double(q[0]) @ K.T / 16.0
    e = np.exp(lg - lg.max(1, keepdims=True))
    e[:, 0] *= 2
    assert np.array_equal(c[0], orc.bf16_from_double((e / e.sum(1, keepdims=True)) @ K[:, :512]))
    # nothing valid -> zeros and lse = -inf
    d, ld = orc.sparse_mla(q, z, p, pt, cache, np.full((1, 8), -1, np.int32))
    assert not d.any() and np.all(np.isneginf(ld))
