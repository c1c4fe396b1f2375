"""GPU parity of the chunked prefill of one long prompt ("GLM-5.3 推理全链路(一)", the
scheduling passage on chunked prefill for 1M contexts, 32K chunks; "GLM-5.3 推理全链路(十一)",
section on the logits temporary and its row chunking): each chunk's rows score every visible
key of the request's index-K cache, select their top-2048 and attend over it, with the logits
scratch bounded by a budget so the indexer runs in row chunks.

Small config: every row's logits and top-k set against the oracle, attention on sampled rows.
Full size (1,048,576 tokens, 32 chunks of 32,768 rows): sampled rows of the first, a middle and
the last chunk, the layer run exactly as the benchmark runs it (4 GiB logits budget).
"""
import numpy as np
import pytest
import torch

import dsa_inputs as gi
import oracle as orc
from parity import (SM, assert_attention_close, assert_logits_close, oracle_index_cache_of, oracle_latent_cache_of,
                    row_queries, topk_sets_match)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402
from sparse_attention_store_amd.workload import DeviceLayer  # noqa: E402

FULL_BUDGET = 4 << 30


def host(t):
    return t.cpu().numpy()


def take(t, rows):
    return host(t[torch.as_tensor(np.asarray(rows), dtype=torch.long, device=t.device)])


def check_rows(w, L, rows, cache, pt, mla_rows=None):
    """Rows of one chunk: q quantisation bit-exact, logits within tolerance (scored again for
    just these rows), top-k sets equal to the oracle's (near-ties excepted), attention of the
    `mla_rows` subset against the oracle over the oracle's selection."""
    rows = np.asarray(sorted(set(int(r) for r in rows)))
    dev = L.q8.device
    ri = torch.as_tensor(rows, dtype=torch.long, device=dev)
    pos = w.row_pos[rows]
    q, wt, qm = row_queries(w, rows, [0])
    q8, qs = orc.quant_fp8(q.reshape(-1, 128))
    assert np.array_equal(host(L.q8[ri]).reshape(-1, 128), q8)
    assert np.array_equal(host(L.qs[ri]).reshape(-1), qs)
    req0 = np.zeros(len(rows), np.int32)
    ref = orc.indexer_logits(q8.reshape(-1, 32, 128), qs.reshape(-1, 32), wt, req0, pos, pt, cache)
    ridx, kth = orc.topk(ref, pos, 2048)
    gidx = host(L.idx[ri])
    topk_sets_match(gidx, ridx, ref, kth)
    long_rows = pos + 1 > 2048
    if long_rows.any():
        sub = ri[torch.as_tensor(np.nonzero(long_rows)[0], device=dev)]
        rws = dsa.Rows(L.rows.req[sub].contiguous(), L.rows.pos[sub].contiguous(), int(pos[long_rows].max()), 1)
        lg = torch.empty((int(long_rows.sum()), dsa.dsa_logits_stride(int(pos[long_rows].max()))),
                         dtype=torch.float32, device=dev)
        dsa.dsa_indexer_logits(L.q8[sub].contiguous(), L.qs[sub].contiguous(), L.w_head[sub].contiguous(), rws,
                               L.pages, L.index_cache[0], lg)
        torch.cuda.synchronize()
        g = host(lg)
        ow = min(ref.shape[1], g.shape[1])
        assert_logits_close(g[:, :ow], ref[long_rows][:, :ow])
    if mla_rows is not None:
        # several top-k sets are correct where scores tie within the tolerance; the set the GPU
        # chose has just been validated, and attention over a given set is unique: the oracle
        # attends over the GPU's selection
        sel = np.isin(rows, mla_rows)
        lat, _ = oracle_latent_cache_of(w, 0, 0, gidx[sel])
        out, lse = orc.sparse_mla(qm[0][sel], req0[sel], pos[sel], pt, lat, gidx[sel], SM)
        assert_attention_close(host(L.out[0][ri])[sel], out)
        assert np.allclose(host(L.lse[0][ri])[sel], lse, rtol=1e-4, atol=1e-4)


def test_small_chunked_prefill_every_row():
    print("\n[gpu] chunked prefill, small: 9000 tokens in chunks of 3100, row-chunked indexer", flush=True)
    w = gi.config(5, "small")
    cache, pt = oracle_index_cache_of(w, 0)
    stride = dsa.dsa_logits_stride(w.max_pos)
    budget = 700 * stride * 4                 # 700 rows of logits per indexer launch
    rng = np.random.default_rng(5)
    base = None
    for c in range((w.R + w.extra["chunk"] - 1) // w.extra["chunk"]):
        wc = gi.prefill_chunk(w, c)
        L = DeviceLayer(wc, latent_layers=[0], logits_budget_bytes=budget, caches_from=base)
        base = base or L
        assert L.row_chunks is not None and len(L.row_chunks) >= 2
        L.full_layer(0)
        torch.cuda.synchronize()
        mla = rng.choice(wc.R, 40, replace=False)
        check_rows(wc, L, np.arange(wc.R), cache, pt, mla_rows=np.concatenate([mla, [0, wc.R - 1]]))
    dsa.dsa_check_device_errors()


def test_full_chunked_prefill_1m_sampled_rows():
    print("\n[gpu] chunked prefill 1M: chunks 0, 15, 31 of 32 x 32768 rows, sampled rows", flush=True)
    w = gi.config(5, "full")
    cache, pt = oracle_index_cache_of(w, 0)
    base = None
    rng = np.random.default_rng(55)
    for c in (0, 15, 31):
        wc = gi.prefill_chunk(w, c)
        L = DeviceLayer(wc, latent_layers=[0], logits_budget_bytes=FULL_BUDGET, caches_from=base)
        base = base or L
        L.full_layer(0)
        torch.cuda.synchronize()
        print(f"[gpu]   chunk {c}: rows {wc.row0}..{wc.row0 + wc.R - 1}, {len(L.row_chunks or [0])} indexer launches",
              flush=True)
        rows = np.concatenate([[0, wc.R - 1], rng.choice(wc.R, 3, replace=False)])
        check_rows(wc, L, rows, cache, pt, mla_rows=rows)
        if L is not base:
            del L
    dsa.dsa_check_device_errors()
    del base
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
