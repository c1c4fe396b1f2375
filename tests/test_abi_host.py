"""C ABI: the library loads and exports every symbol include/dsa.h declares; host-side argument
validation and pure host logic (layer rule, stride, chunking) — no GPU needed."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from sparse_attention_store_amd import dsa
    return dsa


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 14
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(lib.EXPORTED)
    assert lib.abi_version() == 1


def test_mtp_carry_helpers_match_oracle(lib, orc):
    for topk, kpool in [(2048, 1), (2048, 4), (8, 1), (1, 1)]:
        assert lib.dsa_mtp_seed_width(topk, kpool) == orc.mtp_seed_width(topk, kpool)
    assert lib.dsa_mtp_seed_width(0, 1) == -1 and lib.dsa_mtp_seed_width(4096, 1) == -1
    assert lib.dsa_mtp_seed_width(2048, 0) == -1
    for t in (1, 2, 4):
        assert lib.dsa_mtp_carry_allowed(t) == int(orc.mtp_carry_allowed(t))
    assert lib.dsa_mtp_carry_allowed(0) == -1


def test_layer_rule_matches_oracle(lib, orc):
    for kw in [dict(topk_freq=4, skip_topk_offset=3), dict(topk_freq=4), dict(cli_factor=3),
               dict(topk_pattern="FSSFSF"), dict(indexer_types="FFFSSSF")]:
        okw = dict(kw)
        if "topk_pattern" in okw:
            okw["pattern"] = okw.pop("topk_pattern")
        for l in range(80):
            assert lib.dsa_layer_is_shared(l, **kw) == orc.layer_is_shared(l, **okw), (kw, l)


def test_topk_direct_limit_setter(lib):
    default = lib.dsa_set_topk_direct_limit(-1)
    assert default == 1 << 22
    assert lib.dsa_set_topk_direct_limit(0) == default
    assert lib.dsa_set_topk_direct_limit(-5) == 0
    assert lib.dsa_set_topk_direct_limit(default) == 0
    assert lib.dsa_set_topk_direct_limit(-1) == default


def test_stride_and_chunking(lib, orc):
    for p in [0, 1, 254, 255, 256, 4095, 131071, 1048575]:
        assert lib.dsa_logits_stride(p) == orc.logits_stride(p)
    for args in [(10, 100, 1000), (10, 100, 500), (10, 100, 50), (3, 100, 250), (8192, 294912, 1 << 30)]:
        r = orc.logits_rows_per_chunk(*args)
        assert lib.dsa_logits_rows_per_chunk(*args) == (0 if r is None else r)


def _expect(lib, status, fn, *a, **k):
    with pytest.raises(lib.DsaError) as e:
        fn(*a, **k)
    assert e.value.status == status, str(e.value)


class _Fake:
    """Stands in for a device tensor in calls that fail validation before any launch."""
    def __init__(self, ptr, shape=(1,), itemsize=1, strides=None):
        self.ptr, self.shape, self._n, self._is = ptr, shape, 1, itemsize
        for s in shape:
            self._n *= s
        if strides is None:
            strides = tuple(int(__import__("math").prod(shape[i + 1:])) for i in range(len(shape)))
        self._st = strides

    def dim(self):
        return len(self.shape)

    def stride(self, i):
        return self._st[i]

    def data_ptr(self):
        return self.ptr

    def numel(self):
        return self._n

    def element_size(self):
        return self._is


def test_argument_errors(lib):
    import torch
    req = _Fake(0x1000, (4,), 4)
    pos = _Fake(0x2000, (4,), 4)
    rows = lib.Rows(req, pos, max_pos=4095, group=1)
    pt = lib.Pages(_Fake(0x3000, (1, 64), 4), num_pages=64)
    logits = _Fake(0x4000, (4, 4096), 4)
    idx = _Fake(0x5000, (4, 2048), 4)
    # k out of range
    _expect(lib, 1, lib.dsa_topk, logits, rows, 0, idx, _Fake(0x6000, (1 << 20,)))
    _expect(lib, 1, lib.dsa_topk, logits, rows, 4096, idx, _Fake(0x6000, (1 << 20,)))
    # workspace too small
    _expect(lib, 3, lib.dsa_topk, logits, rows, 2048, idx, _Fake(0x6000, (16,)))
    # logits stride too small for max_pos
    small = _Fake(0x4000, (4, 2048), 4)
    _expect(lib, 1, lib.dsa_indexer_logits, _Fake(0x7000), _Fake(0x7100), _Fake(0x7200), rows, pt,
            _Fake(0x8000), small)
    # group must divide n
    bad = lib.Rows(req, pos, max_pos=4095, group=3)
    _expect(lib, 1, lib.dsa_indexer_logits, _Fake(0x7000), _Fake(0x7100), _Fake(0x7200), bad, pt,
            _Fake(0x8000), logits)
    # page table too narrow for max_pos
    narrow = lib.Pages(_Fake(0x3000, (1, 8), 4), num_pages=64)
    _expect(lib, 1, lib.dsa_latent_store, _Fake(0x9000), rows, narrow, _Fake(0xA000))
    # misaligned cache pointer
    _expect(lib, 1, lib.dsa_latent_store, _Fake(0x9000), rows, pt, _Fake(0xA001))
    # null pointers
    _expect(lib, 1, lib.dsa_sparse_mla_decode, _Fake(0), rows, pt, _Fake(0xA000), idx, _Fake(0xB000))
    _expect(lib, 1, lib.dsa_quant_fp8, _Fake(0, (128,)), _Fake(0xC000), _Fake(0xD000))
    # bad sm_scale
    _expect(lib, 1, lib.dsa_sparse_mla_decode, _Fake(0x9000), rows, pt, _Fake(0xA000), idx, _Fake(0xB000),
            sm_scale=0.0)
    # fused norm + RoPE + dual write
    kv = _Fake(0x9000, (4, 576), 2)
    fused = lib.dsa_fused_norm_rope_store
    _expect(lib, 1, fused, kv, rows, pt, None)                                   # no latent cache
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000), index_cache=_Fake(0xE000))  # index without k_idx
    _expect(lib, 1, fused, _Fake(0x9000, (4, 520), 2), rows, pt, _Fake(0xA000))      # row stride < 576
    _expect(lib, 1, fused, _Fake(0x9000, (4, 576), 2, (580, 1)), rows, pt, _Fake(0xA000))  # stride % 8
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000), gamma=_Fake(0xF008))       # misaligned gamma
    q_ok = (64 * 576, 576, 1)
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000), q_pe=_Fake(0x10008 + 1024, (4, 64, 64), 2, q_ok))
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000),
            q_pe=_Fake(0x10000, (4, 64, 64), 2, (60 * 576, 576, 1)))                # rows overlap
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000), q_pe=_Fake(0x10000, (4, 64, 64), 2, (64 * 48, 48, 1)))
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000), rms_eps=-1.0)
    _expect(lib, 1, fused, kv, rows, pt, _Fake(0xA000), index_rope_theta=0.0)
    # reference-rate probes: sizes that are not whole 16-B chunks, misaligned or null pointers
    _expect(lib, 1, lib.dsa_probe_stream_read, _Fake(0x1000, (20,), 1), _Fake(0x2000))
    _expect(lib, 1, lib.dsa_probe_stream_read, _Fake(0x1008, (64,), 1), _Fake(0x2000))
    _expect(lib, 1, lib.dsa_probe_stream_read, _Fake(0x1000, (64,), 1), _Fake(0))
    _expect(lib, 1, lib.dsa_probe_gather_records, _Fake(0x1000, (6560,), 1), 650, _Fake(0x2000, (4,), 4), _Fake(0x3000))
    _expect(lib, 1, lib.dsa_probe_gather_records, _Fake(0x1000, (6560,), 1), 656, _Fake(0x2002, (4,), 4), _Fake(0x3000))
    # a shared layer (no index-K cache) makes store and logits a successful no-op
    lib.dsa_index_k_store(_Fake(0x9000), rows, pt, None)
    lib.dsa_indexer_logits(_Fake(0x7000), _Fake(0x7100), _Fake(0x7200), rows, pt, None, logits)
