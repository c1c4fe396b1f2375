"""dsa_sparse_mla_decode_noalloc (the allocation-free variant, scratch in a fixed device array)
against dsa_sparse_mla_decode on the same inputs, through the C ABI: two calls in a row, the
second with fewer rows, then a one-row call.  256 rows or more run the same stream-K schedule
as the workspace entry point (bit-identical results); fewer rows may run in fewer splits
(within the attention tolerance)."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
from parity import assert_attention_close

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402
from sparse_attention_store_amd.workload import DeviceLayer  # noqa: E402

DEV = "cuda"


def _rows(L, n):
    return dsa.Rows(L.rows.req[:n], L.rows.pos[:n], int(L.w.row_pos[:n].max()), L.w.rows_per_req)


def _idx(w, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((w.R, k), -1, np.int32)
    for r in range(w.R):
        p = int(w.row_pos[r])
        sel = rng.choice(p + 1, size=min(k, p + 1), replace=False)
        idx[r, :len(sel)] = sel
    idx[5, 100:] = -1                      # a row with few keys
    return torch.from_numpy(idx).to(DEV)


def _compare(L, idx, n, exact):
    k = idx.shape[1]
    q = L.q_mla[0][:n]
    ref = torch.empty((n, 64, 512), dtype=torch.int16, device=DEV)
    ref_lse = torch.empty((n, 64), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(dsa.dsa_sparse_mla_workspace_size(n, k), 256), dtype=torch.uint8, device=DEV)
    dsa.dsa_sparse_mla_decode(q, _rows(L, n), L.pages, L.latent_cache[0], idx[:n], ref, ref_lse, ws)
    out = torch.full((n, 64, 512), 0x7FC0, dtype=torch.int16, device=DEV)
    lse = torch.full((n, 64), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_sparse_mla_decode_noalloc(q, _rows(L, n), L.pages, L.latent_cache[0], idx[:n], out, lse)
    torch.cuda.synchronize()
    g, r = out.cpu().numpy(), ref.cpu().numpy()
    gl, rl = lse.cpu().numpy(), ref_lse.cpu().numpy()
    if exact:
        assert np.array_equal(g, r) and np.array_equal(gl, rl)
    else:
        assert_attention_close(g, r)
        assert np.allclose(gl, rl, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("k", [2048, 500])
def test_noalloc_mla_matches_workspace_entry_point(k):
    print(f"\n[gpu] sparse MLA, allocation-free entry point, k={k}", flush=True)
    w = gi.make_decode("noalloc", gi.SEED_BASE + 90, [3000 + 53 * b for b in range(50)], rows_per_req=6)
    assert w.R == 300
    L = DeviceLayer(w, latent_layers=[0])
    idx = _idx(w, k, 90 + k)
    _compare(L, idx, 300, exact=True)      # stream-K: the whole fixed array
    _compare(L, idx, 96, exact=False)      # then fewer rows: splits capped to the array
    _compare(L, idx, 1, exact=False)
    dsa.dsa_check_device_errors()
