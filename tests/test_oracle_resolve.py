"""Pins of the oracle's RESOLVE against things other than itself.

Rules: HiSparse summary page (marsggbo.github.io, 2026-09-23), sections 3-5
(hit detection, LRU eviction, hits to MRU with misses right after, slot vector
aligned with the selection, state updated in place). The pins are an
independent recency-list brute force (tests/brute.py), a hand-worked trace,
state invariants, closed forms and the offline-optimal lower bound.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from tests.brute import BruteLRU, belady_misses, check_invariants, lru_misses
from tiered_kv_cache_hs_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(trace, B, ctx, rows=False, rec=8):
    buf = oracle.OracleBuffer(B, rec, with_rows=rows)
    pool = None
    if rows:
        pool = np.arange(ctx * rec, dtype=np.uint32).astype(np.uint8).reshape(ctx, rec)
        pool = (np.arange(ctx)[:, None] * 7 + np.arange(rec)[None, :]).astype(np.uint8)
    out = []
    for sel in trace:
        s, m = oracle.resolve(buf, np.asarray(sel), pool, ctx)
        out.append((s, m))
    return buf, out


def test_hand_worked_trace():
    g = json.load(open(os.path.join(GOLDEN, "lru_hand_worked.json")))
    buf = oracle.OracleBuffer(g["B"], 4, with_rows=False)
    for st in g["steps"]:
        slots, miss = oracle.resolve(buf, np.array(st["topk"]), None, g["pool_len"])
        assert slots.tolist() == st["slots"]
        assert miss == st["miss"]
        assert buf.pos.tolist() == st["pos"]
        assert buf.stamp.tolist() == st["stamp"]
        assert int(buf.clock[0]) == st["clock"]
        assert int(buf.err[0]) == st["err"]


def _compare_with_brute(trace, B, ctx):
    buf = oracle.OracleBuffer(B, 4, with_rows=False)
    br = BruteLRU(B)
    for sel in trace:
        before = set(int(p) for p in buf.pos if p >= 0)
        slots, miss = oracle.resolve(buf, np.asarray(sel, dtype=np.int32), None, ctx)
        bslots, bmiss, bev = br.step(list(sel))
        assert miss == bmiss
        after = set(int(p) for p in buf.pos if p >= 0)
        assert after == br.resident()
        assert sorted(before - after) == sorted(bev)
        assert slots.tolist() == bslots


def test_brute_force_random_tiny_traces():
    rng = np.random.default_rng(12345)
    n = 0
    for _ in range(10000):
        ctx = int(rng.integers(2, 65))
        k = int(rng.integers(1, min(8, ctx) + 1))
        B = int(rng.integers(k, 17))
        T = int(rng.integers(1, 9))
        # mix fresh random sets with drifting ones so hits are common
        trace = []
        prev = None
        for _t in range(T):
            if prev is not None and rng.random() < 0.7:
                keep = list(rng.permutation(prev)[: int(rng.integers(0, k + 1))])
                pool = [p for p in range(ctx) if p not in keep]
                new = list(rng.choice(pool, size=k - len(keep), replace=False))
                sel = [int(x) for x in rng.permutation(keep + new)]
            else:
                sel = [int(x) for x in rng.choice(ctx, size=k, replace=False)]
            trace.append(sel)
            prev = sel
        _compare_with_brute(trace, B, ctx)
        n += 1
    assert n == 10000


def test_brute_force_exhaustive_ctx5_k2():
    ctx, k = 5, 2
    sels = list(itertools.permutations(range(ctx), k))
    for B in (2, 3, 4):
        for trace in itertools.product(sels, repeat=3):
            _compare_with_brute(trace, B, ctx)


@pytest.mark.parametrize("wl", [1, 2, 3])
def test_invariants_every_step(wl):
    w = I.workload(wl)
    u = 0
    r, l = w.unit(u)
    steps = min(w.steps, 48)
    tr = I.gen_trace(w, r, l, steps)
    cap = w.capacity(r, steps)
    touched = np.unique(tr.astype(np.int64))
    pool = np.zeros((cap, w.rec_bytes), dtype=np.uint8)
    I.fill_records(w, pool.ctypes.data, r, l, positions=touched)
    buf = oracle.OracleBuffer(w.B[r], w.rec_bytes, with_rows=True)
    seen = set()
    length = w.ctx[r]
    for t in range(steps):
        before = buf.pos.copy()
        seen |= set(tr[t].tolist())
        slots, miss = oracle.resolve(buf, tr[t], pool, length)
        check_invariants(before, buf.pos, buf.stamp, buf.clock[0], tr[t], slots, miss, w.B[r], seen)
        occ = np.nonzero(buf.pos >= 0)[0]
        assert np.array_equal(buf.rows[occ], pool[buf.pos[occ]])
        if w.append:
            length += 1
        if t == 0:
            assert miss == w.k


def test_closed_form_B_equals_k_misses_are_the_drift():
    # B = k holds exactly the previous step's set, so from step 1 on every
    # step misses exactly the positions new to the set
    w = I.workload(2)
    tr = I.gen_trace(w, 0, 0, 40)
    buf = oracle.OracleBuffer(w.k, 8, with_rows=False)
    for t in range(40):
        _, miss = oracle.resolve(buf, tr[t], None, w.capacity(0, 40))
        want = w.k if t == 0 else len(set(tr[t].tolist()) - set(tr[t - 1].tolist()))
        assert miss == want
        if t:
            assert miss == w.n_new


def test_closed_form_large_buffer_misses_first_touches_only():
    rng = np.random.default_rng(7)
    ctx, k, T = 300, 16, 30
    trace = []
    for _ in range(T):
        trace.append(rng.choice(ctx, size=k, replace=False))
    B = 300
    buf = oracle.OracleBuffer(B, 8, with_rows=False)
    seen = set()
    for sel in trace:
        _, miss = oracle.resolve(buf, sel, None, ctx)
        assert miss == len(set(sel.tolist()) - seen)
        seen |= set(sel.tolist())


@pytest.mark.parametrize("wl,B", [(1, 256), (1, 384), (1, 512), (2, 2048), (2, 4096)])
def test_belady_lower_bounds_lru(wl, B):
    w = I.workload(wl)
    steps = 32
    tr = I.gen_trace(w, 0, 0, steps)
    trace = [list(map(int, tr[t])) for t in range(steps)]
    buf = oracle.OracleBuffer(B, 8, with_rows=False)
    lru_total = 0
    for t in range(steps):
        _, miss = oracle.resolve(buf, tr[t], None, w.capacity(0, steps))
        lru_total += miss
    assert lru_total == sum(lru_misses(trace, B))
    assert belady_misses(trace, B) <= lru_total


def test_doubling_B_does_not_increase_lru_misses_on_drift_trace():
    # LRU is a stack algorithm: a larger buffer never misses more
    w = I.workload(1)
    tr = I.gen_trace(w, 0, 0, 32)
    tot = []
    for B in (256, 512, 1024):
        buf = oracle.OracleBuffer(B, 8, with_rows=False)
        s = 0
        for t in range(32):
            s += oracle.resolve(buf, tr[t], None, w.ctx[0])[1]
        tot.append(s)
    assert tot[0] >= tot[1] >= tot[2]


def _state(buf):
    return (buf.pos.copy(), buf.stamp.copy(), int(buf.clock[0]))


def test_data_errors_leave_state_unchanged():
    ctx, B = 64, 8
    buf = oracle.OracleBuffer(B, 8, with_rows=True)
    pool = (np.arange(ctx)[:, None] + np.zeros((1, 8), int)).astype(np.uint8)
    oracle.resolve(buf, np.array([1, 2, 3]), pool, ctx)
    snap = _state(buf)
    rows = buf.rows.copy()
    for bad, bit in (([1, 64, 3], oracle.ERR_RANGE), ([1, -1, 3], oracle.ERR_RANGE),
                     ([4, 5, 4], oracle.ERR_DUP)):
        buf.err[0] = 0
        slots, miss = oracle.resolve(buf, np.array(bad), pool, ctx)
        assert miss == -1 and (slots == -1).all()
        assert int(buf.err[0]) == bit
        p, s, c = _state(buf)
        assert np.array_equal(p, snap[0]) and np.array_equal(s, snap[1]) and c == snap[2]
        assert np.array_equal(buf.rows, rows)
    # both kinds at once set both bits; errors are sticky across a valid call
    buf.err[0] = 0
    oracle.resolve(buf, np.array([70, 70, 5]), pool, ctx)
    assert int(buf.err[0]) == oracle.ERR_RANGE  # out-of-range values are not duplicate-checked
    oracle.resolve(buf, np.array([9, 9, 70]), pool, ctx)
    assert int(buf.err[0]) == oracle.ERR_RANGE | oracle.ERR_DUP
    slots, miss = oracle.resolve(buf, np.array([1, 2, 9]), pool, ctx)
    assert miss == 1 and int(buf.err[0]) == 3


def test_clock_exhaustion_is_a_data_error():
    buf = oracle.OracleBuffer(4, 8, with_rows=False)
    buf.clock[0] = 0x7FFFFFFE
    _, m = oracle.resolve(buf, np.array([1]), None, 8)
    assert m == 1 and int(buf.clock[0]) == 0x7FFFFFFF
    assert int(buf.stamp[buf.pos == 1][0]) == 2 * 0x7FFFFFFF - 1
    _, m = oracle.resolve(buf, np.array([1]), None, 8)
    assert m == -1 and int(buf.err[0]) == oracle.ERR_CLOCK


def test_malformed_calls_raise():
    buf = oracle.OracleBuffer(4, 8, with_rows=False)
    with pytest.raises(ValueError):
        oracle.resolve(buf, np.arange(5), None, 8)  # k > B
    with pytest.raises(ValueError):
        oracle.resolve(buf, np.arange(0), None, 8)  # k = 0


def test_snapshot_restore_is_deterministic():
    w = I.workload(1)
    tr = I.gen_trace(w, 0, 0, 20)
    a = oracle.OracleBuffer(w.B[0], 8, with_rows=False)
    for t in range(10):
        oracle.resolve(a, tr[t], None, w.ctx[0])
    b = a.copy()
    for t in range(10, 20):
        sa = oracle.resolve(a, tr[t], None, w.ctx[0])
        sb = oracle.resolve(b, tr[t], None, w.ctx[0])
        assert np.array_equal(sa[0], sb[0]) and sa[1] == sb[1]
    assert np.array_equal(a.pos, b.pos) and np.array_equal(a.stamp, b.stamp)


def test_growth_matches_brute_force():
    """Growing a buffer mid-trace (oracle.grow) against the recency-list
    model given more free slots at the same step: slots, miss counts,
    resident sets and evictions agree at every step; rows carry over."""
    rng = np.random.default_rng(777)
    for case in range(3000):
        ctx = int(rng.integers(3, 49))
        k = int(rng.integers(1, min(6, ctx) + 1))
        B = int(rng.integers(k, 13))
        T = int(rng.integers(2, 9))
        grow_at = int(rng.integers(1, T))
        new_B = B + int(rng.integers(0, 9))
        buf = oracle.OracleBuffer(B, 4, with_rows=False)
        br = BruteLRU(B)
        prev = None
        for t in range(T):
            if t == grow_at:
                buf = oracle.grow(buf, new_B)
                br.grow(new_B)
                assert buf.B == new_B and (buf.pos[B:] == -1).all() and (buf.stamp[B:] == 0).all()
            if prev is not None and rng.random() < 0.7:
                keep = list(rng.permutation(prev)[: int(rng.integers(0, k + 1))])
                pool = [p for p in range(ctx) if p not in keep]
                new = list(rng.choice(pool, size=k - len(keep), replace=False))
                sel = [int(x) for x in rng.permutation(keep + new)]
            else:
                sel = [int(x) for x in rng.choice(ctx, size=k, replace=False)]
            prev = sel
            before = set(int(p) for p in buf.pos if p >= 0)
            slots, miss = oracle.resolve(buf, np.asarray(sel, dtype=np.int32), None, ctx)
            bslots, bmiss, bev = br.step(sel)
            after = set(int(p) for p in buf.pos if p >= 0)
            assert miss == bmiss and after == br.resident(), (case, t)
            assert sorted(before - after) == sorted(bev) and slots.tolist() == bslots, (case, t)


def test_growth_keeps_rows_and_fills_new_slots_first():
    ctx, rec = 40, 8
    pool = (np.arange(ctx)[:, None] * 7 + np.arange(rec)[None, :]).astype(np.uint8)
    buf = oracle.OracleBuffer(4, rec, with_rows=True)
    for sel in ([1, 2, 3, 4], [5, 6, 1, 2]):
        oracle.resolve(buf, np.array(sel), pool, ctx)
    g = oracle.grow(buf, 7)
    assert np.array_equal(g.rows[:4], buf.rows) and np.array_equal(g.pos[:4], buf.pos)
    assert int(g.clock[0]) == 2
    # three new positions: the three new (empty) slots take them, nothing evicted
    slots, miss = oracle.resolve(g, np.array([10, 11, 12]), pool, ctx)
    assert miss == 3 and sorted(slots.tolist()) == [4, 5, 6]
    assert set(g.pos.tolist()) == {5, 6, 1, 2, 10, 11, 12}
    assert np.array_equal(g.rows[4], pool[10])
    with pytest.raises(ValueError):
        oracle.grow(g, 6)
