"""Pins of the oracle's fp64 attention against things other than itself.

Definition: decode attention of one query over the selected positions; the
HiSparse summary page (marsggbo.github.io, 2026-09-23), section 3, states the
method is exact: attention over the resolved slots equals full-KV attention at
the same positions. Pins: a dense numpy fp64 softmax-attention routine when
every position is selected, k = 1, equal keys, permutation invariance, and
that exactness property.
"""
import numpy as np
import pytest

import oracle
from tiered_kv_cache_hs_amd import inputs as I


def _bf16(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bits, round to nearest even (test-side helper)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _widen(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _dense_numpy(Q, K, V, scale):
    """Q [H][d], K [n][d], V [n][dv] fp64 -> softmax(Q K^T scale) V."""
    S = (Q @ K.T) * scale
    S = S - S.max(axis=1, keepdims=True)
    P = np.exp(S)
    return (P @ V) / P.sum(axis=1, keepdims=True)


def _mha_case(rng, n, Hq, Hkv, D, dtype):
    K = rng.standard_normal((n, Hkv, D))
    V = rng.standard_normal((n, Hkv, D))
    q = rng.standard_normal((Hq, D))
    if dtype == oracle.DT_BF16:
        Kb, Vb, qb = _bf16(K), _bf16(V), _bf16(q)
        rows = np.concatenate([Kb.reshape(n, -1), Vb.reshape(n, -1)], axis=1).view(np.uint8)
        return rows, qb, _widen(Kb), _widen(Vb), _widen(qb)
    K32, V32, q32 = K.astype(np.float32), V.astype(np.float32), q.astype(np.float32)
    rows = np.concatenate([K32.reshape(n, -1), V32.reshape(n, -1)], axis=1).view(np.uint8)
    return rows, q32, K32.astype(np.float64), V32.astype(np.float64), q32.astype(np.float64)


@pytest.mark.parametrize("dtype", [oracle.DT_F32, oracle.DT_BF16])
@pytest.mark.parametrize("Hq,Hkv,D", [(1, 1, 64), (4, 2, 32), (8, 8, 128)])
def test_dense_equivalence_mha(dtype, Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 100 + D + dtype)
    n = 256
    rows, q, K, V, qf = _mha_case(rng, n, Hq, Hkv, D, dtype)
    slots = np.arange(n, dtype=np.int32)
    scale = np.float32(1.0 / np.sqrt(D))
    _, o64 = oracle.attend_mha(q, rows, slots, Hkv, D, dtype, dtype, scale, want64=True)
    g = Hq // Hkv
    for h in range(Hq):
        ref = _dense_numpy(qf[h:h + 1], K[:, h // g, :], V[:, h // g, :], float(scale))[0]
        np.testing.assert_allclose(o64[h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("Dl,Dr", [(32, 8), (512, 64)])
def test_dense_equivalence_latent(Dl, Dr):
    rng = np.random.default_rng(Dl)
    n, Hq = 256, 16
    rec = 0.5 * rng.standard_normal((n, Dl + Dr))
    q = rng.standard_normal((Hq, Dl + Dr))
    rb, qb = _bf16(rec), _bf16(q)
    rows = rb.view(np.uint8)
    scale = np.float32(1.0 / np.sqrt(Dl + Dr))
    _, o64 = oracle.attend_latent(qb, rows, np.arange(n, dtype=np.int32), Dl, Dr,
                                  oracle.DT_BF16, oracle.DT_BF16, scale, want64=True)
    ref = _dense_numpy(_widen(qb), _widen(rb), _widen(rb)[:, :Dl], float(scale))
    np.testing.assert_allclose(o64, ref, rtol=1e-12, atol=1e-13)


def test_k1_returns_the_value_row_exactly():
    rng = np.random.default_rng(3)
    rows, q, K, V, _ = _mha_case(rng, 10, 2, 1, 64, oracle.DT_F32)
    o, o64 = oracle.attend_mha(q, rows, np.array([7], np.int32), 1, 64, 0, 0, 0.125, want64=True)
    assert np.array_equal(o64[0], V[7, 0]) and np.array_equal(o64[1], V[7, 0])
    assert np.array_equal(o[0], V[7, 0].astype(np.float32))


def test_equal_keys_give_the_mean_of_values():
    rng = np.random.default_rng(4)
    n, D = 50, 64
    rows, q, K, V, _ = _mha_case(rng, n, 1, 1, D, oracle.DT_F32)
    r = rows.view(np.float32).reshape(n, 2, D)
    r[:, 0, :] = r[0, 0, :]
    rows = r.reshape(n, -1).view(np.uint8)
    slots = np.arange(n, dtype=np.int32)[::-1].copy()
    _, o64 = oracle.attend_mha(q, rows, slots, 1, D, 0, 0, 0.125, want64=True)
    np.testing.assert_allclose(o64[0], r[:, 1, :].astype(np.float64).mean(axis=0), rtol=1e-13, atol=1e-15)


def test_permutation_invariance():
    rng = np.random.default_rng(5)
    n = 300
    rows, q, *_ = _mha_case(rng, n, 4, 4, 128, oracle.DT_BF16)
    sel = rng.choice(n, size=200, replace=False).astype(np.int32)
    _, a = oracle.attend_mha(q, rows, sel, 4, 128, 1, 1, 0.088, want64=True)
    _, b = oracle.attend_mha(q, rows, rng.permutation(sel).astype(np.int32), 4, 128, 1, 1, 0.088, want64=True)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_invalid_slot_gives_nan():
    rng = np.random.default_rng(6)
    rows, q, *_ = _mha_case(rng, 8, 1, 1, 64, oracle.DT_F32)
    o = oracle.attend_mha(q, rows, np.array([1, 8], np.int32), 1, 64, 0, 0, 0.125)
    assert np.isnan(o).all()
    o = oracle.attend_mha(q, rows, np.array([1, -1], np.int32), 1, 64, 0, 0, 0.125)
    assert np.isnan(o).all()


@pytest.mark.parametrize("wl", [1, 3])
def test_exactness_resolved_rows_equal_pool_at_selection(wl):
    # attention through the buffer's resolved slots equals attention over the
    # authoritative host records at the selected positions, bit for bit
    w = I.workload(wl)
    steps = 12
    tr = I.gen_trace(w, 0, 0, steps)
    pool = np.zeros((w.capacity(0, steps), w.rec_bytes), dtype=np.uint8)
    I.fill_records(w, pool.ctypes.data, 0, 0, positions=np.unique(tr.astype(np.int64)))
    buf = oracle.OracleBuffer(w.B[0], w.rec_bytes)
    for t in range(steps):
        q = I.gen_queries(w, t)[0]
        slots, _ = oracle.resolve(buf, tr[t], pool, w.ctx[0])
        if w.kind == "mha":
            a, a64 = oracle.attend_mha(q, buf.rows, slots, w.n_kv_heads, w.head_dim, w.dtype, w.q_dtype,
                                       w.sm_scale, want64=True)
            b, b64 = oracle.attend_mha(q, pool, tr[t], w.n_kv_heads, w.head_dim, w.dtype, w.q_dtype,
                                       w.sm_scale, want64=True)
        else:
            a, a64 = oracle.attend_latent(q, buf.rows, slots, w.latent_dim, w.rope_dim, w.dtype, w.q_dtype,
                                          w.sm_scale, want64=True)
            b, b64 = oracle.attend_latent(q, pool, tr[t], w.latent_dim, w.rope_dim, w.dtype, w.q_dtype,
                                          w.sm_scale, want64=True)
        assert np.array_equal(a64, b64) and np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_append_writes_pool_only():
    pool = np.zeros((10, 4), dtype=np.uint8)
    length = np.array([6], dtype=np.int64)
    oracle.append(pool, length, 6, np.full((2, 4), 9, np.uint8))
    assert length[0] == 8 and (pool[6:8] == 9).all() and (pool[:6] == 0).all()
    with pytest.raises(ValueError):
        oracle.append(pool, length, 9, np.zeros((1, 4), np.uint8))  # gap past the length
    with pytest.raises(ValueError):
        oracle.append(pool, length, 8, np.zeros((3, 4), np.uint8))  # past capacity
