"""Pins for the oracle's fused norm + RoPE + dual-cache write ("vLLM 推理链路概览", section on
the KV low-rank projection and cache; "GLM-5.3 推理全链路(一)", section 4.3 on the fused_norm_rope
kernel and its has_indexer switch): RMSNorm against NumPy and its closed forms, the rope tail and
the in-place q_pe rotation against complex multiplication, the index-K entry against the
separately pinned store, and what must stay untouched."""
import numpy as np

import dsa_inputs as gi

EPS = 1e-6
LAT_PAGE = 64 * 656


def _bf16(orc, x):
    return orc.bf16_from_double(np.asarray(x, np.float64))


def _setup(orc, n=70, seed=50, pages=4, width=576):
    rng = np.random.default_rng(seed)
    scale = 2.0 ** rng.integers(-6, 6, (n, 1))
    kv = _bf16(orc, rng.standard_normal((n, width)) * scale)
    gamma = _bf16(orc, rng.standard_normal(512) * 0.5 + 1.0)
    pos = (np.arange(n, dtype=np.int32) * 3) % (64 * pages)
    pt = gi.permutation(seed, 9, pages).astype(np.int32)[None, :]
    return rng, kv, gamma, pos, pt


def _record(cache, pt, p):
    page = cache[pt[0, p // 64]]
    return page[(p % 64) * 656:(p % 64 + 1) * 656]


def _np_rmsnorm(c, gamma, eps=EPS):
    return c / np.sqrt(np.mean(c * c) + eps) * gamma


def _np_ue8m0(amax):
    """Smallest power of two s with amax <= 448 s, by search over exponents."""
    e = np.floor(np.log2(amax / 448.0)) - 1
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return 2.0 ** e


def _np_rope(v, p, theta):
    """Rotation of interleaved pairs as complex multiplication by exp(i p theta^(-2i/64))."""
    z = v[0::2] + 1j * v[1::2]
    z = z * np.exp(1j * p * theta ** (-np.arange(32) * 2.0 / 64.0))
    out = np.empty(64)
    out[0::2], out[1::2] = z.real, z.imag
    return out


def _bf16_close(orc, got_bits, ref):
    """bf16 bits equal the rounding of ref, or ref sits within 1e-12 of the midpoint between the
    two neighbouring bf16 values (where the order of double operations may decide)."""
    got = orc.bf16_to_double(got_bits)
    want = orc.bf16_to_double(_bf16(orc, ref))
    bad = got != want
    if bad.any():
        mid = (got[bad] + want[bad]) / 2
        assert np.all(np.abs(ref[bad] - mid) <= 1e-12 * np.abs(ref[bad])), \
            f"{bad.sum()} bf16 values differ beyond a near-tie: {got[bad][:4]} vs {want[bad][:4]}"


def test_rmsnorm_record_against_numpy(orc):
    rng, kv, gamma, pos, pt = _setup(orc)
    cache = np.zeros((pt.shape[1], LAT_PAGE), np.uint8)
    orc.fused_norm_rope_store(kv, np.zeros(len(pos), np.int32), pos, pt, cache, gamma=gamma)
    g = orc.bf16_to_double(gamma)
    for t in range(len(pos)):
        rec = _record(cache, pt, int(pos[t]))
        y = _np_rmsnorm(orc.bf16_to_double(kv[t, :512]), g)
        for b in range(4):
            blk = y[128 * b:128 * b + 128]
            s = _np_ue8m0(np.abs(blk).max())
            assert rec[512 + 4 * b:516 + 4 * b].view(np.float32)[0] == s
            codes = rec[128 * b:128 * b + 128]
            assert np.array_equal(codes, orc.fp8_encode(blk / s)), (t, b)
            # dequantised within half an e4m3 step of the normalised value
            deq = orc.fp8_decode(codes) * s
            half = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(blk / s), 2.0 ** -6))) - 4), 2.0 ** -10)
            assert np.all(np.abs(deq - blk) <= half * s * (1 + 1e-12))


def test_rmsnorm_closed_forms(orc):
    rng, kv, gamma, pos, pt = _setup(orc, n=40, seed=51)
    req = np.zeros(len(pos), np.int32)
    base = np.zeros((pt.shape[1], LAT_PAGE), np.uint8)
    orc.fused_norm_rope_store(kv, req, pos, pt, base, rms_eps=0.0)
    # eps = 0: RMSNorm is invariant under an exact power-of-two scaling of the input
    scaled = _bf16(orc, orc.bf16_to_double(kv) * 2.0 ** 5)
    c2 = np.zeros_like(base)
    orc.fused_norm_rope_store(np.concatenate([scaled[:, :512], kv[:, 512:]], 1), req, pos, pt, c2, rms_eps=0.0)
    assert np.array_equal(c2, base)
    # gamma = 2 everywhere doubles every block scale and leaves the codes alone
    c3 = np.zeros_like(base)
    orc.fused_norm_rope_store(kv, req, pos, pt, c3, gamma=_bf16(orc, np.full(512, 2.0)), rms_eps=0.0)
    for t in range(len(pos)):
        r0, r3 = _record(base, pt, int(pos[t])), _record(c3, pt, int(pos[t]))
        assert np.array_equal(r3[:512], r0[:512]) and np.array_equal(r3[528:], r0[528:])
        assert np.array_equal(r3[512:528].view(np.float32), 2 * r0[512:528].view(np.float32))
    # a constant vector a normalises to a / sqrt(a^2 + eps): 1 - eps / (2 a^2) to first order
    a = 0.75
    const = kv.copy()
    const[:, :512] = _bf16(orc, np.full(512, a))
    c4 = np.zeros_like(base)
    orc.fused_norm_rope_store(const, req, pos, pt, c4, rms_eps=0.01)
    v = a / np.sqrt(a * a + 0.01)
    s = _np_ue8m0(v)
    rec = _record(c4, pt, int(pos[0]))
    assert np.all(rec[:512] == orc.fp8_encode(np.array([v / s]))[0])
    assert np.all(rec[512:528].view(np.float32) == s)


def test_rope_tail_is_a_complex_rotation(orc):
    rng, kv, gamma, pos, pt = _setup(orc, n=64, seed=52)
    pos[:8] = np.arange(8)                         # includes p = 0
    pos[8:] = 1_000_000 - np.arange(56) * 997      # large angles: evaluated in double
    pt = np.zeros((1, 1_000_000 // 64 + 1), np.int32)
    used = np.unique(pos // 64)
    pt[0, used] = gi.permutation(52, 9, len(used)).astype(np.int32)   # a small pool for the pages in use
    cache = np.zeros((len(used), LAT_PAGE), np.uint8)
    orc.fused_norm_rope_store(kv, np.zeros(64, np.int32), pos, pt, cache, theta=50000.0)
    for t in range(64):
        p = int(pos[t])
        tail = _record(cache, pt, p)[528:].view(np.uint16)
        kr = orc.bf16_to_double(kv[t, 512:576])
        if p == 0:
            assert np.array_equal(tail, kv[t, 512:576])
        _bf16_close(orc, tail, _np_rope(kr, p, 50000.0))
        back = _np_rope(orc.bf16_to_double(tail), -p, 50000.0)
        assert np.all(np.abs(back - kr) <= 2.0 ** -7 * np.max(np.abs(kr)))


def test_q_pe_rotated_in_place(orc):
    rng, kv, gamma, pos, pt = _setup(orc, n=9, seed=53)
    pos[4] = -1                                     # padded: q row untouched too
    q = _bf16(orc, rng.standard_normal((9, 64, 576)))
    q0 = q.copy()
    cache = np.zeros((pt.shape[1], LAT_PAGE), np.uint8)
    orc.fused_norm_rope_store(kv, np.zeros(9, np.int32), pos, pt, cache, q=q, q_off=512, theta=20000.0)
    assert np.array_equal(q[:, :, :512], q0[:, :, :512])
    assert np.array_equal(q[4], q0[4])
    for t in range(9):
        if pos[t] < 0:
            continue
        for h in range(64):
            _bf16_close(orc, q[t, h, 512:], _np_rope(orc.bf16_to_double(q0[t, h, 512:]), int(pos[t]), 20000.0))
    # a contiguous [n, 64, 64] q_pe gives the same rotation
    qc = np.ascontiguousarray(q0[:, :, 512:])
    orc.fused_norm_rope_store(kv, np.zeros(9, np.int32), pos, pt, np.zeros_like(cache), q=qc, theta=20000.0)
    assert np.array_equal(qc, q[:, :, 512:])


def test_index_entry_equals_the_separate_store(orc):
    rng, kv, gamma, pos, pt = _setup(orc, n=100, seed=54)
    k_idx = _bf16(orc, rng.standard_normal((100, 128)) * 2 + 0.5)
    req = np.zeros(100, np.int32)
    lat = np.zeros((pt.shape[1], LAT_PAGE), np.uint8)
    idx = np.full((pt.shape[1], 8448), 0xCD, np.uint8)
    orc.fused_norm_rope_store(kv, req, pos, pt, lat, index_cache=idx, k_idx=k_idx, gamma=gamma,
                              theta=50000.0, index_theta=10000.0, ln_eps=1e-5)
    ref = np.full_like(idx, 0xCD)
    orc.index_k_store(k_idx, req, pos, pt, ref, eps=1e-5, theta=10000.0)
    assert np.array_equal(idx, ref)
    # the latent records do not depend on whether the index entry is written
    lat2 = np.zeros_like(lat)
    orc.fused_norm_rope_store(kv, req, pos, pt, lat2, gamma=gamma, theta=50000.0)
    assert np.array_equal(lat, lat2)


def test_untouched_without_indexer_or_position(orc):
    rng, kv, gamma, pos, pt = _setup(orc, n=20, seed=55)
    k_idx = _bf16(orc, rng.standard_normal((20, 128)))
    pos[3] = -1
    req = np.zeros(20, np.int32)
    idx = np.full((pt.shape[1], 8448), 0x5A, np.uint8)
    lat = np.full((pt.shape[1], LAT_PAGE), 0x5A, np.uint8)
    orc.fused_norm_rope_store(kv, req, pos, pt, lat, index_cache=None, k_idx=k_idx)
    assert np.all(idx == 0x5A)                      # a shared layer writes no index-K
    written = {int(p) for p in pos if p >= 0}
    for p in range(64 * pt.shape[1]):
        rec = _record(lat, pt, p)
        assert np.all(rec == 0x5A) == (p not in written), p


def test_kv_row_stride(orc):
    """kv may be the latent part of the A projection's output row ([n, 2048 + 576])."""
    rng, kv, gamma, pos, pt = _setup(orc, n=30, seed=56)
    wide = _bf16(orc, rng.standard_normal((30, 2048 + 576)))
    wide[:, 2048:] = kv
    a = np.zeros((pt.shape[1], LAT_PAGE), np.uint8)
    b = np.zeros_like(a)
    orc.fused_norm_rope_store(kv, np.zeros(30, np.int32), pos, pt, a, gamma=gamma)
    orc.fused_norm_rope_store(wide, np.zeros(30, np.int32), pos, pt, b, gamma=gamma, kv_off=2048)
    assert np.array_equal(a, b)
