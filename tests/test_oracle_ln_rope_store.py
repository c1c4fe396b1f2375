"""Pins for LayerNorm, interleaved RoPE and the two cache stores (closed forms, invariants,
an independent complex-number formulation, and byte-layout checks)."""
import numpy as np

import dsa_inputs as gi


def test_layernorm_closed_form(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)) * rng.uniform(0.01, 5, (50, 1)) + rng.uniform(-3, 3, (50, 1))
    y = orc.ln_rope(x, 0, eps=1e-6)          # RoPE at position 0 is the identity
    var = x.var(1)
    assert np.allclose(y.mean(1), 0, atol=1e-12)
    assert np.allclose(y.var(1), var / (var + 1e-6), rtol=1e-12)


def test_rope_matches_complex_rotation(orc):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((20, 128))
    pos = rng.integers(0, 1 << 20, 20)
    y = orc.ln_rope(x, pos, ln=False)
    z = x[:, 0:64:2] + 1j * x[:, 1:64:2]
    freqs = 10000.0 ** (-np.arange(32) / 32.0)
    zr = z * np.exp(1j * pos[:, None] * freqs[None, :])
    assert np.allclose(y[:, 0:64:2], zr.real, atol=1e-9) and np.allclose(y[:, 1:64:2], zr.imag, atol=1e-9)
    assert np.array_equal(y[:, 64:], x[:, 64:])


def test_rope_group_properties(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((10, 128))
    assert np.array_equal(orc.ln_rope(x, 0, ln=False), x)
    p = rng.integers(0, 1 << 20, 10)
    y = orc.ln_rope(x, p, ln=False)
    assert np.allclose(np.linalg.norm(y[:, :64], axis=1), np.linalg.norm(x[:, :64], axis=1), rtol=1e-12)
    assert np.allclose(orc.ln_rope(y, p, ln=False, inverse=True), x, atol=1e-9)
    q = rng.integers(0, 1000, 10)
    assert np.allclose(orc.ln_rope(orc.ln_rope(x, p, ln=False), q, ln=False), orc.ln_rope(x, p + q, ln=False), atol=1e-8)
    # relative-position property: <R_p a, R_q b> depends only on p - q
    a, b = x[0:1], x[1:2]
    d1 = (orc.ln_rope(a, 1000, ln=False) * orc.ln_rope(b, 700, ln=False))[:, :64].sum()
    d2 = (orc.ln_rope(a, 5300, ln=False) * orc.ln_rope(b, 5000, ln=False))[:, :64].sum()
    assert abs(d1 - d2) < 1e-9


def _tiny_pages(n_tokens, seed=11):
    ctx = np.array([n_tokens])
    pt = gi.permutation(seed, 9, (n_tokens + 63) // 64).astype(np.int32)[None, :]
    return pt


def test_index_k_store_layout(orc):
    n = 200                                   # 4 pages, ragged last page
    pt = _tiny_pages(n)
    k = gi.normal_bf16(1, 2, 0, n * 128).reshape(n, 128)
    pos = np.arange(n, dtype=np.int32)
    pos[7] = -1                               # a padded row writes nothing
    cache = np.zeros((pt.shape[1] + 1, 8448), np.uint8)
    pre = orc.index_k_store(k, np.zeros(n, np.int32), pos, pt, cache, want_pre=True)
    y = orc.ln_rope(orc.bf16_to_double(k), np.arange(n))
    for p in [0, 63, 64, 150, 199]:
        page, slot = pt[0, p // 64], p % 64
        codes = cache[page, slot * 128:(slot + 1) * 128]
        s = cache[page, 8192 + 4 * slot:8192 + 4 * slot + 4].view(np.float32)[0]
        assert s == orc.ue8m0(np.abs(y[p]).max()[None])[0]
        assert np.array_equal(codes, orc.fp8_encode(y[p] / s, brute=True))
        assert np.allclose(pre[p], y[p] / s, rtol=0, atol=0)
        # dequantised key is within half an fp8 ulp (relative 2^-4) of LN+RoPE(x)
        deq = orc.fp8_decode(codes) * s
        assert np.all(np.abs(deq - y[p]) <= np.maximum(np.abs(y[p]) * 2.0 ** -4, s * 2.0 ** -10))
    page7, slot7 = pt[0, 0], 7
    assert not cache[page7, slot7 * 128:(slot7 + 1) * 128].any()
    assert not cache[-1].any()                # a page nobody owns stays untouched


def test_index_k_store_page_permutation_invariance(orc):
    n = 256
    k = gi.normal_bf16(2, 2, 0, n * 128).reshape(n, 128)
    pos = np.arange(n, dtype=np.int32)
    out = []
    for seed in (1, 2):
        pt = _tiny_pages(n, seed)
        cache = np.zeros((4, 8448), np.uint8)
        orc.index_k_store(k, np.zeros(n, np.int32), pos, pt, cache)
        logical = np.stack([np.concatenate([cache[pt[0, p // 64], (p % 64) * 128:(p % 64 + 1) * 128],
                                            cache[pt[0, p // 64], 8192 + 4 * (p % 64):8196 + 4 * (p % 64)]])
                            for p in range(n)])
        out.append(logical)
    assert np.array_equal(out[0], out[1])


def test_latent_store_layout(orc):
    n = 130
    pt = _tiny_pages(n, 3)
    kv = gi.normal_bf16(3, 5, 0, n * 576).reshape(n, 576)
    cache = np.zeros((pt.shape[1], 64 * 656), np.uint8)
    orc.latent_store(kv, np.zeros(n, np.int32), np.arange(n, dtype=np.int32), pt, cache)
    x = orc.bf16_to_double(kv)
    for p in [0, 64, 129]:
        rec = cache[pt[0, p // 64], (p % 64) * 656:(p % 64 + 1) * 656]
        for b in range(4):
            s = rec[512 + 4 * b:516 + 4 * b].view(np.float32)[0]
            blk = x[p, 128 * b:128 * (b + 1)]
            assert s == orc.ue8m0(np.abs(blk).max()[None])[0]
            assert np.array_equal(rec[128 * b:128 * (b + 1)], orc.fp8_encode(blk / s, brute=True))
        assert np.array_equal(rec[528:656].view(np.uint16), kv[p, 512:])
