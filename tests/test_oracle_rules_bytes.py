"""Pins for the full/shared layer rule and the byte accounting against the numbers printed
on the pages (tests/golden/*)."""
import json
import math
import os

import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _full_list():
    with open(os.path.join(GOLD, "glm53_full_layers.txt")) as f:
        return [int(t) for line in f if not line.startswith("#") for t in line.split()]


def test_glm53_rule_freq_offset(orc):
    full = [l for l in range(78) if not orc.layer_is_shared(l, topk_freq=4, skip_topk_offset=3)]
    assert full == _full_list()
    assert len(full) == 21 and 78 - len(full) == 57


def test_glm53_explicit_list_wins(orc):
    types = ["full" if l in _full_list() else "shared" for l in range(78)]
    assert [orc.layer_is_shared(l, indexer_types=types, cli_factor=3, topk_freq=1) for l in range(78)] == \
        [l not in _full_list() for l in range(78)]
    assert orc.layer_is_shared(200, indexer_types=types) is False     # beyond the list: full


def test_default_offset_two(orc):
    # offset 2: layers 0 and 1 full, layer 2 skipped, then one full layer in every 4
    full = [l for l in range(20) if not orc.layer_is_shared(l, topk_freq=4)]
    assert full == [0, 1, 5, 9, 13, 17]


def test_cli_factor_and_pattern(orc):
    assert [orc.layer_is_shared(l, cli_factor=3) for l in range(7)] == [False, True, True, False, True, True, False]
    assert [orc.layer_is_shared(l, pattern="FSSF") for l in range(6)] == [False, True, True, False, False, False]
    assert [orc.layer_is_shared(l, topk_freq=1) for l in range(5)] == [False] * 5


def _gold():
    with open(os.path.join(GOLD, "page_numbers.json")) as f:
        return {it["name"]: it for it in json.load(f)["items"]}


def _close(name, v):
    g = _gold()[name]
    assert abs(v - g["value"]) <= g["tol"] * abs(g["value"]) + 1e-12, (name, v, g)


def test_bytes_against_pages(orc):
    _close("index_k_bytes_per_token", orc.index_k_bytes_per_token())
    _close("index_k_page_bytes", orc.index_k_page_bytes())
    _close("latent_bytes_per_token", orc.latent_bytes_per_token())
    _close("latent_bytes_78_layers_per_token", 78 * orc.latent_bytes_per_token())
    _close("read_per_layer_L1e5", orc.read_bytes_per_full_layer(10 ** 5))
    _close("read_per_step_L1e5", orc.read_bytes_per_step(10 ** 5))
    _close("read_per_layer_L1e5_MiB", orc.read_bytes_per_full_layer(10 ** 5) / 2 ** 20)
    _close("read_per_step_L1e5_MiB", orc.read_bytes_per_step(10 ** 5) / 2 ** 20)
    _close("read_per_layer_L1e6", orc.read_bytes_per_full_layer(10 ** 6))
    _close("read_per_step_L1e6", orc.read_bytes_per_step(10 ** 6))
    _close("t_idx_h200_ms", orc.index_read_seconds(1, 10 ** 5, 4.8e12) * 1e3)
    _close("t_idx_h100_ms", orc.index_read_seconds(1, 10 ** 5, 3.35e12) * 1e3)
    _close("index_read_b32_L1e5", 32 * orc.read_bytes_per_step(10 ** 5))
    _close("index_read_b4_L1e6", 4 * orc.read_bytes_per_step(10 ** 6))
    _close("write_per_step", orc.write_bytes_per_step())
    _close("logits_b32_L1e5", orc.logits_bytes(32, 10 ** 5))
    _close("logits_b32_L1e6", orc.logits_bytes(32, 10 ** 6))
    _close("logits_row_bytes_L100", orc.logits_bytes(1, 100))
    _close("logits_row_bytes_L2048", orc.logits_bytes(1, 2048))
    _close("pd_index_cache_1M", orc.index_pool_bytes(21, 2 ** 20))
    _close("pd_latent_1M", 78 * orc.latent_bytes_per_token() * 2 ** 20)
    _close("indexer_q_bytes_per_token", orc.indexer_q_bytes_per_token())
    _close("block_table_bytes_L1e5", orc.block_table_bytes(10 ** 5))
    _close("troubleshoot_read_1M_bytes", 2.6 * orc.read_bytes_per_full_layer(10 ** 6))
    _close("troubleshoot_read_1M_ms", 2.6 * orc.read_bytes_per_full_layer(10 ** 6) / 4.8e12 * 1e3)
    _close("mtp_layer_read_1M", orc.read_bytes_per_full_layer(10 ** 6))
    _close("mxfp4_index_bytes_per_token", 128 // 2 + 128 // 32)
    _close("mla_flops_per_token_layer", 2 * 64 * 512 * 2048)
    _close("mtp_seed_width", orc.mtp_seed_width(2048, 1))
    _close("mtp_saved_read_per_132L", orc.mtp_carry_saved_read_bytes(1000) / (132 * 1000))
    _close("mtp_saved_fraction", orc.mtp_carry_saved_fraction())


def test_chunked_prefill_accounting(orc):
    # the page's 1M prefill scoring figure, ~94 PFLOP over 21 layers, is the closed form
    _close("prefill_1m_indexer_flops", orc.chunked_prefill_indexer_flops())
    # its ~47 TB read figure does not state the read granularity; one read of the visible keys per
    # 32 query rows lands on it.  32 is a reading fitted to that figure, so this is a consistency
    # check of the reading, not a pin of the helper (the limits below pin the helper)
    _close("prefill_1m_indexer_read_bytes", orc.chunked_prefill_indexer_read_bytes(1 << 20, 32))
    # the read formula's limits: one row per block reads every row's own prefix ...
    L = 1000
    assert orc.chunked_prefill_indexer_read_bytes(L, 1, 1) == 132 * L * (L + 1) // 2
    # ... and one block covering the prompt reads it once
    assert orc.chunked_prefill_indexer_read_bytes(L, L, 1) == 132 * L
    assert orc.chunked_prefill_indexer_read_bytes(L, 4 * L, 1) == 132 * L
    # brute force on a tiny prompt: rows 0..L-1 each score i + 1 keys; blocks read their prefix
    L, block = 10, 4
    assert orc.chunked_prefill_indexer_flops(L, 1, 1, 1) == 2 * sum(i + 1 for i in range(L))
    assert orc.chunked_prefill_indexer_read_bytes(L, block, 1) == 132 * (4 + 8 + 10)
    # the reads grow with the square of the prompt: twice the blocks, about four times the bytes
    r1 = orc.chunked_prefill_indexer_read_bytes(1 << 20, 32768, 1)
    r2 = orc.chunked_prefill_indexer_read_bytes(1 << 21, 32768, 1)
    assert 3.9 < r2 / r1 < 4.0
    # one read per 32K chunk: 48 GB over 21 layers, a thousandth of the 32-row accounting
    assert orc.chunked_prefill_indexer_read_bytes(1 << 20, 32768) == 21 * 132 * 32768 * 528


def test_mtp_carry_rule(orc):
    # only a single draft chain may carry the seed; a kpool > 1 widens it by the tail slots
    assert orc.mtp_carry_allowed(1) and not orc.mtp_carry_allowed(2) and not orc.mtp_carry_allowed(4)
    assert orc.mtp_seed_width(2048, 4) == 2051


def test_rows_per_chunk_rule(orc):
    f = orc.logits_rows_per_chunk
    assert f(10, 100, 1000) is None          # fits the budget: no chunking
    assert f(10, 100, 500) == 5
    assert f(10, 100, 50) == 1               # at least one row
    assert f(3, 100, 250) == 2
    assert f(2, 100, 150) == 1
