"""GPU parity of the fused norm + RoPE + dual-cache write ("vLLM 推理链路概览", section on the KV
low-rank projection and cache; "GLM-5.3 推理全链路(一)", section 4.3 on fused_norm_rope and its
has_indexer switch) against the CPU oracle on the same seeded inputs: latent records, index-K
entries and the in-place query rotation, all byte for byte."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import LN_EPS, THETA

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402

DEV = "cuda"
RMS_EPS = 1e-6
MLA_THETA = 50000.0          # a different base from the indexer's, so a swap would show


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy()


def _inputs(seed, n, q_width=576):
    kv = gi.normal_bf16(seed, gi.T_KV_A, 0, n * gi.KV_A_WIDTH).reshape(n, gi.KV_A_WIDTH)
    gamma = gi.normal_bf16(seed, gi.T_GAMMA, 0, 512)
    k_idx = gi.normal_bf16(seed, gi.T_RAW_K, 0, n * 128).reshape(n, 128)
    q = gi.normal_bf16(seed, gi.T_MLA_Q, 0, n * 64 * q_width).reshape(n, 64, q_width)
    return kv, gamma, k_idx, q


def _run_both(req, pos, page_table, num_pages, kv, gamma, k_idx, q, q_off, indexer=True, kv_off=2048,
              max_pos=None):
    n = len(pos)
    lat_ref = np.zeros((num_pages, 41984), np.uint8)
    idx_ref = np.full((num_pages, 8448), 0x5A, np.uint8)
    q_ref = q.copy() if q is not None else None
    orc.fused_norm_rope_store(kv, req, pos, page_table, lat_ref, index_cache=idx_ref if indexer else None,
                              k_idx=k_idx, gamma=gamma, q=q_ref, q_off=q_off, rms_eps=RMS_EPS, ln_eps=LN_EPS,
                              theta=MLA_THETA, index_theta=THETA, kv_off=kv_off)
    lat = torch.zeros((num_pages, 41984), dtype=torch.uint8, device=DEV)
    idx = torch.full((num_pages, 8448), 0x5A, dtype=torch.uint8, device=DEV)
    dkv = dev(kv.view(np.int16))
    dq = dev(q.view(np.int16)) if q is not None else None
    mp = int(pos.max()) if max_pos is None else max_pos
    rows = dsa.Rows(dev(req), dev(pos), max(mp, 0), 1)
    pages = dsa.Pages(dev(page_table), num_pages)
    dsa.dsa_fused_norm_rope_store(dkv[:, kv_off:kv_off + 576] if kv_off else dkv, rows, pages, lat,
                                  index_cache=idx if indexer else None,
                                  k_idx=dev(k_idx.view(np.int16)) if indexer else None,
                                  gamma=dev(gamma.view(np.int16)) if gamma is not None else None,
                                  q_pe=dq[:, :, q_off:q_off + 64] if dq is not None else None,
                                  rms_eps=RMS_EPS, ln_eps=LN_EPS, rope_theta=MLA_THETA, index_rope_theta=THETA)
    torch.cuda.synchronize()
    dsa.dsa_check_device_errors()
    return (host(lat), lat_ref), (host(idx), idx_ref), ((host(dq).view(np.uint16), q_ref) if q is not None else None)


def _same(pair, what):
    got, ref = pair
    diff = np.argwhere(got != ref)
    assert len(diff) == 0, f"{what}: {len(diff)} elements differ, first at {diff[:5].tolist()}"


@pytest.mark.parametrize("cid", [0, 1, 2, 4])
def test_fused_store_bit_exact(cid):
    print(f"\n[gpu] fused norm+rope store c{cid}", flush=True)
    w = gi.config(cid, "small")
    pos = w.row_pos.copy()
    if len(pos) > 4:
        pos[len(pos) // 2] = -1                      # a padded token: nothing written, q untouched
    kv, gamma, k_idx, q = _inputs(w.seed, w.R)
    lat, idx, qq = _run_both(w.row_req, pos, w.page_table, w.num_pages, kv, gamma, k_idx, q, 512,
                             max_pos=int(w.row_pos.max()))
    _same(lat, "latent cache")
    _same(idx, "index-K cache")
    _same(qq, "q")


def test_fused_store_without_indexer_gamma_or_q():
    print("\n[gpu] fused store, latent only", flush=True)
    w = gi.config(1, "small")
    kv, _, k_idx, _ = _inputs(w.seed + 1, w.R)
    lat, idx, _ = _run_both(w.row_req, w.row_pos, w.page_table, w.num_pages, np.ascontiguousarray(kv[:, 2048:]),
                            None, k_idx, None, 0, indexer=False, kv_off=0)
    _same(lat, "latent cache")
    assert np.all(idx[0] == 0x5A)                    # no index write without an index cache


def test_fused_store_large_positions():
    """Positions near 1M: the angles (up to 1e6 rad) are evaluated in double on both sides."""
    print("\n[gpu] fused store near position 1M", flush=True)
    pos = (1_000_000 - np.arange(256) * 997).astype(np.int32)
    pt = np.zeros((1, 1_000_000 // 64 + 1), np.int32)
    used = np.unique(pos // 64)
    pt[0, used] = gi.permutation(77, gi.T_PERM, len(used)).astype(np.int32)
    kv, gamma, k_idx, q = _inputs(77, 256, q_width=64)
    lat, idx, qq = _run_both(np.zeros(256, np.int32), pos, pt, len(used), kv, gamma, k_idx, q, 0)
    _same(lat, "latent cache")
    _same(idx, "index-K cache")
    _same(qq, "q")


def test_fused_index_entry_equals_separate_store():
    print("\n[gpu] fused vs separate index-K store", flush=True)
    w = gi.config(4, "small")
    kv, gamma, k_idx, q = _inputs(w.seed, w.R)
    rows = dsa.Rows(dev(w.row_req), dev(w.row_pos), int(w.row_pos.max()), 1)
    pages = dsa.Pages(dev(w.page_table), w.num_pages)
    a = torch.zeros((w.num_pages, 8448), dtype=torch.uint8, device=DEV)
    b = torch.zeros_like(a)
    lat = torch.zeros((w.num_pages, 41984), dtype=torch.uint8, device=DEV)
    dk = dev(k_idx.view(np.int16))
    dsa.dsa_fused_norm_rope_store(dev(kv.view(np.int16))[:, 2048:], rows, pages, lat, index_cache=a, k_idx=dk,
                                  ln_eps=LN_EPS, index_rope_theta=THETA)
    dsa.dsa_index_k_store(dk, rows, pages, b, LN_EPS, THETA)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_fused_store_full_size_prefill_chunk():
    """The chunked-prefill chunk at full size: 8192 new tokens on a 65,536-token prefix, with the
    index-K entry and the query rotation, every byte compared."""
    print("\n[gpu] fused store c4 full size", flush=True)
    w = gi.config(4, "full")
    kv, gamma, k_idx, q = _inputs(w.seed, w.R, q_width=64)
    lat, idx, qq = _run_both(w.row_req, w.row_pos, w.page_table, w.num_pages, kv, gamma, k_idx, q, 0)
    _same(lat, "latent cache")
    _same(idx, "index-K cache")
    _same(qq, "q")


def test_fused_store_empty_and_all_padded():
    """No tokens: a successful no-op.  Every token padded: nothing written, q left as it was."""
    print("\n[gpu] fused store, empty and all-padded batches", flush=True)
    w = gi.config(0, "small")
    kv, gamma, k_idx, q = _inputs(w.seed, 4)
    pages = dsa.Pages(dev(w.page_table), w.num_pages)
    lat = torch.full((w.num_pages, 41984), 0x5A, dtype=torch.uint8, device=DEV)
    idx = torch.full((w.num_pages, 8448), 0x5A, dtype=torch.uint8, device=DEV)
    dq = dev(q.view(np.int16))
    q0 = dq.clone()
    empty = dsa.Rows(torch.zeros(0, dtype=torch.int32, device=DEV), torch.zeros(0, dtype=torch.int32, device=DEV), 0, 1)
    dsa.dsa_fused_norm_rope_store(dev(kv.view(np.int16))[:0, 2048:], empty, pages, lat, index_cache=idx,
                                  k_idx=dev(k_idx.view(np.int16))[:0], gamma=dev(gamma.view(np.int16)))
    padded = dsa.Rows(dev(np.zeros(4, np.int32)), dev(np.full(4, -1, np.int32)), 0, 1)
    dsa.dsa_fused_norm_rope_store(dev(kv.view(np.int16))[:, 2048:], padded, pages, lat, index_cache=idx,
                                  k_idx=dev(k_idx.view(np.int16)), gamma=dev(gamma.view(np.int16)),
                                  q_pe=dq[:, :, 512:])
    torch.cuda.synchronize()
    assert bool((lat == 0x5A).all()) and bool((idx == 0x5A).all()) and torch.equal(dq, q0)
    dsa.dsa_check_device_errors()
