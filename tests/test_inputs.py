"""Properties of the seeded input generators (traces, records, queries)."""
import dataclasses

import numpy as np
import pytest

from tiered_kv_cache_hs_amd import inputs as I


@pytest.mark.parametrize("wl", [1, 2, 3, 4, 5, 6, 7])
def test_trace_properties(wl):
    w = I.workload(wl)
    steps = min(w.steps, 24)
    r, l = w.unit(w.n_units - 1)
    tr = I.gen_trace(w, r, l, steps)
    assert tr.shape == (steps, w.k) and tr.dtype == np.int32
    for t in range(steps):
        s = tr[t]
        length = w.ctx[r] + (t if w.append else 0)
        assert len(np.unique(s)) == w.k
        assert s.min() >= 0 and s.max() < length
        if t:
            assert len(set(s.tolist()) - set(tr[t - 1].tolist())) == w.n_new
    assert np.array_equal(tr, I.gen_trace(w, r, l, steps))  # reproducible


def test_trace_streams_differ_per_unit_and_prefix_stable():
    w = I.workload(4)
    a, b = I.gen_trace(w, 0, 0, 8), I.gen_trace(w, 0, 1, 8)
    assert not np.array_equal(a, b)
    assert np.array_equal(I.gen_trace(w, 0, 0, 4), a[:4])


def test_workload_shapes():
    assert [I.workload(i).n_new for i in (1, 2, 3, 4, 5, 6, 7)] == [26, 266, 266, 143, 614, 266, 67]
    assert [I.workload(i).rec_bytes for i in range(1, 8)] == [512, 4096, 1152, 4096, 1152, 1152,
                                                              1152]
    w7 = I.workload(7)  # compressed entries: 512 of 32768 / 4 per step
    assert (w7.k, w7.ctx[0], w7.B[0], w7.n_requests) == (512, 8192, 1024, 32)
    w5 = I.workload(5)
    assert all(16384 <= c < 1048576 for c in w5.ctx) and set(w5.B) <= {2048, 4096, 8192}
    assert len(set(w5.B)) == 3


def test_recency_source_leans_to_the_end():
    w = I.workload(2)
    tr = I.gen_trace(w, 0, 0, 64)
    new = np.concatenate([np.setdiff1d(tr[t], tr[t - 1]) for t in range(1, 64)])
    # Zipf(1.1) over the distance from the end; recent positions already in
    # the set are rejected, yet accepted picks stay far more recent than a
    # uniform draw (median distance ~ half the context)
    assert np.median(w.ctx[0] + 64 - new) < w.ctx[0] / 4


@pytest.mark.parametrize("wl", [1, 3])
def test_record_fill_is_order_and_layout_independent(wl):
    w = I.workload(wl)
    pos = np.array([0, 17, 4095, 5, 1000], dtype=np.int64)
    full = np.zeros((4096, w.rec_bytes), np.uint8)
    I.fill_records(w, full.ctypes.data, 0, 0, p0=0, p1=4096)
    sparse = np.zeros((4096, w.rec_bytes), np.uint8)
    I.fill_records(w, sparse.ctypes.data, 0, 0, positions=pos[::-1].copy())
    assert np.array_equal(full[pos], sparse[pos])
    assert np.array_equal(I.record_array(w, 0, 0, pos), full[pos])
    vals = full.view(np.float32 if w.dtype == I.F32 else np.uint16)
    if w.dtype == I.BF16:
        vals = I.bf16_bits_to_f32(vals)
    assert abs(float(vals.std()) - w.rec_sigma) < 0.02 * w.rec_sigma


def test_queries_shape_and_steps_differ():
    w = I.workload(3)
    a, b = I.gen_queries(w, 0), I.gen_queries(w, 1)
    assert a.shape == (8, 64, 576) and a.dtype == np.uint16
    assert not np.array_equal(a, b)


def test_layer_groups_reuse_one_selection():
    w = I.workload(6)
    assert (w.n_requests, w.n_layers, w.share, w.k, w.rec_bytes) == (8, 8, 4, 2048, 1152)
    assert [w.group_base(l) for l in range(8)] == [0, 0, 0, 0, 4, 4, 4, 4]
    tr = I.gen_traces(dataclasses.replace(w, n_requests=2, ctx=w.ctx[:2], B=w.B[:2]), 6)
    for r in range(2):
        for l in range(8):
            g = w.group_base(l)
            assert np.array_equal(tr[:, r * 8 + l], tr[:, r * 8 + g])
        assert not np.array_equal(tr[:, r * 8], tr[:, r * 8 + 4])  # groups differ
    assert np.array_equal(tr[:, 4], I.gen_trace(w, 0, 4, 6))  # a group's trace is its first layer's
    # records still differ per layer
    a, b = I.record_array(w, 0, 0, [5]), I.record_array(w, 0, 1, [5])
    assert not np.array_equal(a, b)
