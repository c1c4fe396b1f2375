"""The benchmark's reference-rate probes read every byte they are given: the XOR of the words
each work-group folds into its sink word, taken over the whole sink, equals the XOR of every
32-bit word of the data, computed on the host.  Cases: a streaming read of a ragged buffer, and a
gather of whole records, 656-B latent records and another size (with repeated and out-of-pool
ids, which the gather clamps into the pool)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_attention_store_amd import dsa  # noqa: E402


def _xor_words(a: np.ndarray) -> int:
    return int(np.bitwise_xor.reduce(np.ascontiguousarray(a).view(np.uint32).ravel(), initial=np.uint32(0)))


@pytest.mark.parametrize("nbytes", [16, 4096, 1_000_000 * 16 + 48])
def test_stream_read_probe_reads_every_word(nbytes):
    print(f"\n[gpu] stream-read probe {nbytes} B", flush=True)
    rng = np.random.default_rng(nbytes)
    h = rng.integers(0, 256, nbytes, dtype=np.uint8)
    buf = torch.from_numpy(h).cuda()
    sink = torch.full((dsa.PROBE_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    dsa.dsa_probe_stream_read(buf, sink)
    torch.cuda.synchronize()
    assert _xor_words(sink.cpu().numpy()) == _xor_words(h)


@pytest.mark.parametrize("rec", [656, 64])
def test_gather_probe_reads_every_record(rec):
    print(f"\n[gpu] gather probe, {rec}-B records", flush=True)
    rng = np.random.default_rng(7)
    n_rec = 5000
    pool = rng.integers(0, 256, n_rec * rec, dtype=np.uint8)
    ids = rng.integers(0, n_rec, 12_345).astype(np.int32)
    ids[:3] = [-5, n_rec + 9, ids[5]]          # clamped to record 0, record n_rec - 1, and a repeat
    sink = torch.full((dsa.PROBE_SINK_WORDS,), -1, dtype=torch.int32, device="cuda")
    dsa.dsa_probe_gather_records(torch.from_numpy(pool).cuda(), rec, torch.from_numpy(ids).cuda(), sink)
    torch.cuda.synchronize()
    recs = pool.reshape(n_rec, rec)[np.clip(ids, 0, n_rec - 1)]
    assert _xor_words(sink.cpu().numpy()) == _xor_words(recs)
