"""The oracle's batched step (oracle_step_batch, timed as the CPU baseline)
does exactly the work of the per-unit calls: for every unit, resolve then
attention, with the same slots, miss counts, buffer state, rows and outputs,
bit for bit, whatever the thread count. Its team size is set per call and
does not change the process-wide OpenMP setting."""
import numpy as np
import pytest

import oracle
from tiered_kv_cache_hs_amd import inputs as I


def _units(w, bufs, pools, lens, traces, t, q, slots, miss, out):
    units = []
    for u in range(w.n_units):
        b = bufs[u]
        x = oracle.OracleUnitC()
        x.B, x.k = b.B, w.k
        x.pos, x.stamp, x.clock = b.pos.ctypes.data, b.stamp.ctypes.data, b.clock.ctypes.data
        x.err, x.rows, x.rec_bytes = b.err.ctypes.data, b.rows.ctypes.data, w.rec_bytes
        x.pool, x.pool_len = pools[u].ctypes.data, lens[u]
        x.topk = traces[t, u].ctypes.data
        x.slots, x.miss = slots[u].ctypes.data, miss[u:].ctypes.data
        x.kind = 0 if w.kind == "mha" else 1
        x.Hq, x.Hkv, x.D, x.Dl, x.Dr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.latent_dim, w.rope_dim
        x.kv_dtype, x.q_dtype, x.sm_scale = w.dtype, w.q_dtype, np.float32(w.sm_scale)
        x.q, x.out = q[u].ctypes.data, out[u].ctypes.data
        units.append(x)
    return units


def _compare(w, steps, n_threads):
    traces = I.gen_traces(w, steps)
    pools, lens, A, Bf = {}, {}, {}, {}
    for u in range(w.n_units):
        r, l = divmod(u, w.n_layers)
        pool = np.zeros((w.capacity(r, steps), w.rec_bytes), np.uint8)
        pos = np.unique(traces[:, u, :].astype(np.int64))
        I.fill_records(w, pool.ctypes.data, r, l, positions=pos[pos < w.ctx[r]])
        pools[u], lens[u] = pool, w.ctx[r]
        A[u] = oracle.OracleBuffer(w.B[r], w.rec_bytes)
        Bf[u] = oracle.OracleBuffer(w.B[r], w.rec_bytes)
    n = w.n_units
    for t in range(steps):
        q = I.gen_queries(w, t)
        slots = np.full((n, w.k), -7, np.int32)
        miss = np.full(n, -7, np.int32)
        out = np.full((n, w.n_q_heads, w.out_dim), np.nan, np.float32)
        used = oracle.step_batch(_units(w, A, pools, lens, traces, t, q, slots, miss, out),
                                 n_threads)
        assert 1 <= used <= n
        for u in range(n):
            so, mo = oracle.resolve(Bf[u], traces[t, u], pools[u], lens[u])
            assert np.array_equal(slots[u], so), (t, u)
            assert miss[u] == mo, (t, u)
            for f in ("pos", "stamp", "clock", "err", "rows"):
                assert np.array_equal(getattr(A[u], f), getattr(Bf[u], f)), (t, u, f)
            if w.kind == "mha":
                want = oracle.attend_mha(q[u], Bf[u].rows, so, w.n_kv_heads, w.head_dim, w.dtype,
                                         w.q_dtype, np.float32(w.sm_scale))
            else:
                want = oracle.attend_latent(q[u], Bf[u].rows, so, w.latent_dim, w.rope_dim,
                                            w.dtype, w.q_dtype, np.float32(w.sm_scale))
            assert np.array_equal(out[u].view(np.uint32), want.view(np.uint32)), (t, u)


@pytest.mark.parametrize("n_threads", [0, 1, 3])
def test_step_batch_equals_per_unit_calls_tiny_workload(n_threads):
    _compare(I.workload(1), 32, n_threads)


def test_step_batch_equals_per_unit_calls_batch8_latent_units():
    """Workload 3's units (batch 8, latent records, k 2048, B 4096) at its
    full shapes, over its first steps (the cold step and warm ones)."""
    _compare(I.workload(3), 3, 0)


def test_step_batch_leaves_the_process_thread_setting_alone():
    import ctypes
    import ctypes.util
    gomp = ctypes.CDLL(ctypes.util.find_library("gomp") or "libgomp.so.1")
    before = gomp.omp_get_max_threads()
    w = I.workload(1)
    _compare(w, 2, 1)
    assert gomp.omp_get_max_threads() == before
