"""End-to-end closed form of one DSA layer in the oracle: index-K store -> q quantisation ->
indexer logits -> top-k -> latent store -> sparse MLA.

Keys planted along the query's weighted indexer direction are the exact top-k set (the needle
construction of the indexer pins), and the latent records at those positions all hold one vector
v.  Softmax over equal logits weighs every selected record by 1/k, so each head's output is v
itself and its log-normaliser is the common logit plus ln k.  Any wrong selection, page lookup or
normalisation moves the output off v: the latent records elsewhere are random."""
import numpy as np

import dsa_inputs as gi

L, K, SEED = 6000, 512, 99
SM_SCALE = 1.0 / 16.0


def _layer(orc, swap_one=False):
    pt = gi.permutation(SEED, 9, (L + 63) // 64).astype(np.int32)[None, :]
    req = np.zeros(L, np.int32)
    pos = np.arange(L, dtype=np.int32)
    row_pos = np.array([L - 1], np.int32)

    # indexer: needles along the weighted query direction, as the indexer pins build them
    q = gi.normal_bf16(SEED, 1, 0, 32 * 128).reshape(1, 32, 128)
    q8, qs = orc.quant_fp8(q.reshape(32, 128))
    w = gi.uniform_f32(SEED, 3, 0, 32, gi.w_scale()).reshape(1, 32)
    u = (orc.fp8_decode(q8) * qs[:, None] * w[0][:, None]).sum(0)
    needles = gi.choose_distinct(SEED, 11, L - 1, K)
    raw = gi.normal_bf16(SEED, 2, 0, L * 128).reshape(L, 128)
    d = orc.ln_rope(np.repeat(u[None], K, 0), needles, ln=False, inverse=True)
    d -= d.mean(1, keepdims=True)
    d *= np.sqrt(128) / np.linalg.norm(d, axis=1, keepdims=True)
    raw[needles] = orc.bf16_from_double(d)
    icache = np.zeros((pt.shape[1], orc.IDX_PAGE_BYTES), np.uint8)
    orc.index_k_store(raw, req, pos, pt, icache)
    lg = orc.indexer_logits(q8[None], qs[None], w, np.zeros(1, np.int32), row_pos, pt, icache)
    idx, _ = orc.topk(lg, row_pos, K)

    # latent cache: random records, the same 576-dim row at every needle
    kv = gi.normal_bf16(SEED, 4, 0, L * 576).reshape(L, 576)
    kv[needles] = gi.normal_bf16(SEED, 5, 0, 576)[None]
    lcache = np.zeros((pt.shape[1], orc.LAT_PAGE_BYTES), np.uint8)
    orc.latent_store(kv, req, pos, pt, lcache)

    if swap_one:
        # one selected slot points at a random record instead of a needle
        other = np.setdiff1d(np.arange(L - 1), needles)[0]
        idx = idx.copy()
        idx[0, 0] = other
    qm = gi.normal_bf16(SEED, 6, 0, 64 * 576).reshape(1, 64, 576)
    out, lse = orc.sparse_mla(qm, np.zeros(1, np.int32), row_pos, pt, lcache, idx, SM_SCALE)
    return needles, idx, pt, lcache, qm, out, lse


def _record(orc, pt, lcache, s):
    """Decoded 576-dim key of position s: four scaled FP8 blocks, then the bf16 rope tail."""
    page = lcache[pt[0, s // 64]]
    rec = page[(s % 64) * 656:(s % 64 + 1) * 656]
    sc = rec[512:528].view(np.float32)
    c = orc.fp8_decode(rec[:512]).astype(np.float64) * np.repeat(sc.astype(np.float64), 128)
    kr = orc.bf16_to_double(rec[528:656].view(np.uint16))
    return np.concatenate([c, kr])


def test_layer_closed_form(orc):
    needles, idx, pt, lcache, qm, out, lse = _layer(orc)
    assert np.array_equal(idx[0], needles)
    key = _record(orc, pt, lcache, int(needles[0]))
    for s in needles[1:]:
        assert np.array_equal(_record(orc, pt, lcache, int(s)), key)
    # every head returns the common value vector, rounded once to bf16
    v = orc.bf16_from_double(key[:512])
    assert np.array_equal(out[0], np.broadcast_to(v, (64, 512)))
    # and its log-normaliser is the common logit plus ln k
    qd = orc.bf16_to_double(qm[0])
    np.testing.assert_allclose(lse[0], SM_SCALE * (qd @ key) + np.log(K), rtol=1e-6, atol=1e-6)


def test_layer_closed_form_detects_a_wrong_selection(orc):
    _, _, _, _, _, out, _ = _layer(orc, swap_one=True)
    _, _, pt, lcache, _, ref, _ = _layer(orc)
    assert not np.array_equal(out, ref)
