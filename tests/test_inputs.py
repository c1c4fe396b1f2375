"""The seeded generator: distribution sanity, determinism, slicing consistency (CPU)."""
import numpy as np

import dsa_inputs as gi


def test_normal_moments_and_range():
    x = gi.bf16_to_f32(gi.normal_bf16(123, 2, 0, 1 << 20)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.var() - 1) < 0.01
    assert np.abs(x).max() <= 6.0


def test_slices_and_gathers_agree():
    a = gi.normal_bf16(5, 7, 1000, 5000)
    b = gi.normal_bf16(5, 7, 3000, 100)
    assert np.array_equal(a[2000:2100], b)
    idx = np.array([1000, 1999, 5999, 4321])
    assert np.array_equal(gi.normal_bf16_at(5, 7, idx), a[idx - 1000])


def test_streams_differ():
    assert not np.array_equal(gi.normal_bf16(5, 1, 0, 64), gi.normal_bf16(5, 2, 0, 64))
    assert not np.array_equal(gi.normal_bf16(5, 1, 0, 64), gi.normal_bf16(6, 1, 0, 64))


def test_uniform():
    u = gi.uniform_f32(9, 3, 0, 100000)
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    w = gi.uniform_f32(9, 3, 0, 10, gi.w_scale())
    assert np.allclose(w, (u[:10].astype(np.float64) / np.sqrt(32)).astype(np.float32), rtol=0, atol=0)


def test_permutation_and_workloads():
    p = gi.permutation(1, 9, 1000)
    assert np.array_equal(np.sort(p), np.arange(1000))
    for cid in range(5):
        w = gi.config(cid, "small")
        used = np.concatenate([w.page_table[b, :(w.ctx[b] + 63) // 64] for b in range(w.B)])
        assert len(np.unique(used)) == len(used) and used.max() < w.num_pages
        assert np.all(w.row_pos < w.ctx[w.row_req])
    w = gi.config(2)
    assert w.R == 384 and w.ctx[0] == 131072 and list(w.row_pos[:6]) == list(range(131066, 131072))
    w = gi.config(1)
    assert w.B == 32 and w.ctx.min() >= 8192 and w.ctx.max() <= 32768
    w = gi.config(3)
    assert w.ctx[0] == 1 << 20 and len(np.unique(w.needles)) == 2048
