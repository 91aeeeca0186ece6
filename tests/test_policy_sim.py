"""The replacement-policy simulator against independent references (CPU).

* its LRU is the oracle's resolve (HiSparse summary, sections 4-5): same
  per-step miss counts on workload traces and random traces;
* its Belady is the exhaustive optimum on tiny traces (every choice of
  victims at every step), and no policy beats it on larger ones;
* Swap-vanilla's misses are the set differences of consecutive selections;
* with a buffer holding every position ever selected, every policy misses
  exactly the first selections of each position.
"""
import itertools

import numpy as np
import pytest

import oracle
from tiered_kv_cache_hs_amd import inputs as I
from tiered_kv_cache_hs_amd import policy_sim as P


def random_trace(rng, T, k, ctx, keep):
    """Drifting selections: keep `keep` of the previous set, draw the rest."""
    cur = rng.choice(ctx, size=k, replace=False)
    out = [cur.copy()]
    for _ in range(T - 1):
        kept = rng.choice(cur, size=keep, replace=False)
        pool = np.setdiff1d(np.arange(ctx), kept)
        cur = np.concatenate([kept, rng.choice(pool, size=k - keep, replace=False)])
        rng.shuffle(cur)
        out.append(cur.copy())
    return np.array(out, dtype=np.int64)


def oracle_lru_misses(trace, B):
    buf = oracle.OracleBuffer(B, 16, with_rows=False)
    out = []
    for t in range(trace.shape[0]):
        _, m = oracle.resolve(buf, trace[t].astype(np.int32), None, int(trace.max()) + 1)
        out.append(m)
    return np.array(out)


@pytest.mark.parametrize("seed,T,k,ctx,keep,B", [(1, 30, 8, 40, 6, 12), (2, 40, 16, 200, 10, 16),
                                                 (3, 25, 32, 120, 20, 80), (4, 60, 5, 9, 3, 7)])
def test_lru_matches_oracle_random(seed, T, k, ctx, keep, B):
    tr = random_trace(np.random.default_rng(seed), T, k, ctx, keep)
    assert np.array_equal(P.misses_lru(tr, B), oracle_lru_misses(tr, B))


def test_lru_matches_oracle_workload1():
    w = I.workload(1)
    tr = I.gen_traces(w, w.steps)[:, 0, :]
    assert np.array_equal(P.misses_lru(tr, w.B[0]), oracle_lru_misses(tr, w.B[0]))


def brute_min_misses(trace, B):
    """Smallest total misses over every victim choice at every step."""
    best = [None]

    def go(t, res, acc):
        if best[0] is not None and acc >= best[0]:
            return
        if t == trace.shape[0]:
            best[0] = acc
            return
        sel = set(int(p) for p in trace[t])
        new = [p for p in sel if p not in res]
        need = len(new) - (B - len(res))
        cand = sorted(p for p in res if p not in sel)
        choices = itertools.combinations(cand, need) if need > 0 else [()]
        for ev in choices:
            go(t + 1, (res - set(ev)) | set(new), acc + len(new))

    go(0, frozenset(), 0)
    return best[0]


@pytest.mark.parametrize("seed", range(12))
def test_belady_is_the_exhaustive_optimum(seed):
    rng = np.random.default_rng(100 + seed)
    k = int(rng.integers(1, 3))
    ctx = int(rng.integers(k + 2, 7))
    B = int(rng.integers(k, min(ctx, k + 3) + 1))
    tr = random_trace(rng, 7, k, ctx, max(0, k - 1))
    assert P.misses_belady(tr, B).sum() == brute_min_misses(tr, B)


@pytest.mark.parametrize("seed", range(4))
def test_no_policy_beats_belady(seed):
    tr = random_trace(np.random.default_rng(200 + seed), 50, 24, 150, 18)
    for B in (24, 36, 60):
        opt = P.misses_belady(tr, B).sum()
        for pol in ("lru", "fifo", "random"):
            assert P.simulate(tr, pol, B, seed=seed).sum() >= opt, (pol, B)


def test_swap_vanilla_is_the_set_difference():
    tr = random_trace(np.random.default_rng(7), 30, 20, 100, 15)
    m = P.misses_swap(tr)
    assert m[0] == 20
    for t in range(1, tr.shape[0]):
        assert m[t] == len(set(tr[t].tolist()) - set(tr[t - 1].tolist()))
    assert np.array_equal(P.simulate(tr, "swap", 20), m)


def test_a_buffer_holding_everything_misses_first_uses_only():
    tr = random_trace(np.random.default_rng(9), 20, 10, 60, 6)
    seen, first = set(), []
    for t in range(tr.shape[0]):
        s = set(tr[t].tolist())
        first.append(len(s - seen))
        seen |= s
    for pol in ("lru", "fifo", "random", "belady"):
        assert np.array_equal(P.simulate(tr, pol, 60), np.array(first)), pol


def test_rejects_bad_traces():
    tr = np.array([[1, 2, 3], [1, 1, 2]])
    with pytest.raises(ValueError):
        P.misses_lru(tr, 4)
    with pytest.raises(ValueError):
        P.misses_fifo(np.array([[1, 2, 3]]), 2)
    with pytest.raises(ValueError):
        P.simulate(np.array([[1, 2]]), "swap", 3)


def test_study_on_a_workload_trace():
    w = I.workload(1)
    tr = I.gen_traces(w, 12)
    rows = P.study(tr)
    rate = {(r["policy"], r["B"] // w.k): r["mean_miss_rate"] for r in rows}
    assert rate[("belady", 2)] <= min(rate[("lru", 2)], rate[("fifo", 2)], rate[("random", 2)])
    assert rate[("lru", 4)] <= rate[("lru", 2)] + 1e-12
    assert all(0.0 <= v <= 1.0 for v in rate.values())


def test_B_sweep_is_monotone_for_belady_and_starts_at_swap():
    """Belady never misses more with a larger buffer (an optimal policy with
    more room can always mimic the smaller one); at B = k every policy is
    Swap-vanilla."""
    w = I.workload(1)
    tr = I.gen_traces(w, 16)
    rows = P.sweep_B(tr, policies=("lru", "belady", "fifo"), mults=(1.0, 1.5, 2.0, 4.0))
    bel = [r["mean_miss_rate"] for r in rows if r["policy"] == "belady"]
    assert all(b1 >= b2 - 1e-12 for b1, b2 in zip(bel, bel[1:]))
    swap = np.mean([P.misses_swap(tr[:, u, :])[1:] / w.k for u in range(tr.shape[1])])
    for r in rows:
        if r["B"] == w.k:
            assert abs(r["mean_miss_rate"] - swap) < 1e-12, r

