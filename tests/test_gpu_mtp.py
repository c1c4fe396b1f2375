"""GPU parity of the MTP draft-step top-k carry ("GLM-5.3 推理全链路(十一)", section 优化三:
MTP 迭代内复用 topk): in a draft iteration, step 0's top-k seed is the oracle's top-k of step 0's
rows; every later step reuses that very tensor (no copy) and its attention equals the oracle's
attention over the seed with the step's own queries; without the carry each step selects its own
top-k."""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import assert_attention_close, oracle_index_cache, oracle_latent_cache, queries, topk_sets_match

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402
from sparse_attention_store_amd.workload import DeviceLayer, SM_SCALE  # noqa: E402


def host(t):
    return t.cpu().numpy()


def _oracle_step(w, st, q8all, qsall, wt, cache):
    g = w.rows_per_req
    sel = np.arange(w.R // g) * g + st
    req = np.arange(len(sel), dtype=np.int32)
    pos = w.row_pos[sel]
    # the steps' rows are one per request: request b's page table row is b
    lg = orc.indexer_logits(q8all[sel], qsall[sel], wt[sel], req, pos, w.page_table, cache)
    idx, kth = orc.topk(lg, pos, 2048)
    return sel, req, pos, lg, idx, kth


@pytest.mark.parametrize("steps", [5])
def test_mtp_carry_reuses_the_step0_seed(steps):
    print("\n[gpu] mtp draft round with carry", flush=True)
    w = gi.config(2, "small")
    D = DeviceLayer(w, latent_layers=[0])
    m = D.mtp_draft_round(carry=True, steps=steps)
    torch.cuda.synchronize()
    q, wt, qm = queries(w, [0])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    q8, qs = q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32)
    cache = oracle_index_cache(w)
    lat = oracle_latent_cache(w, 0)
    sel0, req, pos0, lg0, idx0, kth0 = _oracle_step(w, 0, q8, qs, wt, cache)
    seed = host(m["idx"][0])
    topk_sets_match(seed, idx0, lg0, kth0)
    assert dsa.dsa_mtp_seed_width(2048, 1) == seed.shape[1] and dsa.dsa_mtp_carry_allowed(1) == 1
    for st in range(steps):
        sel = np.arange(w.R // w.rows_per_req) * w.rows_per_req + st
        ref, _ = orc.sparse_mla(qm[0][sel], req, w.row_pos[sel], w.page_table, lat, seed, SM_SCALE)
        assert_attention_close(host(m["out"][st]).view(np.uint16), ref)
    dsa.dsa_check_device_errors()


def test_mtp_without_carry_selects_per_step():
    print("\n[gpu] mtp draft round without carry", flush=True)
    w = gi.config(2, "small")
    D = DeviceLayer(w, latent_layers=[0])
    m = D.mtp_draft_round(carry=False, steps=3)
    torch.cuda.synchronize()
    q, wt, _ = queries(w, [])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    q8, qs = q8.reshape(w.R, 32, 128), qs.reshape(w.R, 32)
    cache = oracle_index_cache(w)
    for st in range(3):
        _, _, _, lg, idx, kth = _oracle_step(w, st, q8, qs, wt, cache)
        topk_sets_match(host(m["idx"][st]), idx, lg, kth)
