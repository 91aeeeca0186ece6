"""Replacement-policy study over top-k selection traces (CPU).

HiSparse summary (marsggbo.github.io, 2026-09-23), section 4: selections of
neighbouring decode steps overlap heavily, and the page compares cache
policies on replayed selection traces at k = 2048: keeping only the current
selection (Swap-vanilla, B = k), LRU, FIFO and random at B = 4096, the
offline optimum (Belady) and LRU at B = 8192, by the mean per-step fraction
of selected positions that miss.

Every policy here serves set requests: at step t the k selected positions
must all be resident afterwards; a miss is a selected position that was not
resident before the step, and a missed position needs a slot, taken from the
residents that step t does not select (B >= k, so one always exists):

* ``lru``   -- the resolve's own rule: the victim is the resident not
  selected at t with the smallest (last-use stamp, position); at step c
  selected hits get stamp 2c and newly fetched positions 2c - 1;
* ``fifo``  -- the resident that entered first (ties: smaller position);
* ``random``-- a uniformly random non-selected resident (seeded);
* ``belady``-- the non-selected resident whose next selection is farthest
  in the future, never-again first (ties: smaller position);
* ``swap``  -- Swap-vanilla: only the current selection is kept (B = k),
  so the misses of step t are the positions new to its selection.

Position order only breaks ties and, unlike slot numbers, does not depend on
how a buffer lays out its slots, so miss counts are layout-independent.

Usage: ``python -m tiered_kv_cache_hs_amd.policy_sim --workload 3`` prints
the study table for a workload's synthetic traces.
"""
from __future__ import annotations

import argparse
import heapq
import time
from typing import Dict, List, Sequence

import numpy as np

POLICIES = ("swap", "lru", "fifo", "random", "belady")


def _check_trace(trace: np.ndarray, B: int) -> None:
    if trace.ndim != 2:
        raise ValueError("trace must be [steps][k]")
    k = trace.shape[1]
    if B < k:
        raise ValueError(f"B = {B} below k = {k}")
    for t in range(trace.shape[0]):
        if len(np.unique(trace[t])) != k:
            raise ValueError(f"step {t} selects a position twice")


def misses_swap(trace: np.ndarray) -> np.ndarray:
    """Swap-vanilla (B = k): the buffer holds exactly the last selection."""
    out = np.empty(trace.shape[0], dtype=np.int64)
    prev: set = set()
    for t in range(trace.shape[0]):
        cur = set(int(p) for p in trace[t])
        out[t] = len(cur - prev)
        prev = cur
    return out


def misses_lru(trace: np.ndarray, B: int) -> np.ndarray:
    """LRU with the resolve's stamps: hits 2c, fetched 2c - 1 at step c."""
    _check_trace(trace, B)
    stamp: Dict[int, int] = {}  # resident position -> last-use stamp
    out = np.empty(trace.shape[0], dtype=np.int64)
    for t in range(trace.shape[0]):
        c = t + 1
        sel = [int(p) for p in trace[t]]
        selset = set(sel)
        new = [p for p in sel if p not in stamp]
        need = len(new) - (B - len(stamp))  # evictions needed
        if need > 0:
            cand = [(s, p) for p, s in stamp.items() if p not in selset]
            for _, p in heapq.nsmallest(need, cand):
                del stamp[p]
        for p in sel:
            stamp[p] = 2 * c if p in stamp else 2 * c - 1
        out[t] = len(new)
    return out


def misses_fifo(trace: np.ndarray, B: int) -> np.ndarray:
    _check_trace(trace, B)
    enter: Dict[int, int] = {}  # resident position -> step it entered
    out = np.empty(trace.shape[0], dtype=np.int64)
    for t in range(trace.shape[0]):
        sel = [int(p) for p in trace[t]]
        selset = set(sel)
        new = [p for p in sel if p not in enter]
        need = len(new) - (B - len(enter))
        if need > 0:
            cand = [(e, p) for p, e in enter.items() if p not in selset]
            for _, p in heapq.nsmallest(need, cand):
                del enter[p]
        for p in new:
            enter[p] = t
        out[t] = len(new)
    return out


def misses_random(trace: np.ndarray, B: int, seed: int = 0) -> np.ndarray:
    _check_trace(trace, B)
    rng = np.random.default_rng(seed)
    res: set = set()
    out = np.empty(trace.shape[0], dtype=np.int64)
    for t in range(trace.shape[0]):
        sel = [int(p) for p in trace[t]]
        selset = set(sel)
        new = [p for p in sel if p not in res]
        need = len(new) - (B - len(res))
        if need > 0:
            cand = np.array(sorted(p for p in res if p not in selset), dtype=np.int64)
            for p in rng.choice(cand, size=need, replace=False):
                res.discard(int(p))
        res.update(new)
        out[t] = len(new)
    return out


def next_use(trace: np.ndarray) -> List[Dict[int, int]]:
    """For every step t, each selected position's next step of selection
    after t (absent: never again)."""
    T = trace.shape[0]
    nxt: List[Dict[int, int]] = [dict() for _ in range(T)]
    upcoming: Dict[int, int] = {}
    for t in range(T - 1, -1, -1):
        for p in trace[t]:
            p = int(p)
            if p in upcoming:
                nxt[t][p] = upcoming[p]
        for p in trace[t]:
            upcoming[int(p)] = t
    return nxt


def misses_belady(trace: np.ndarray, B: int) -> np.ndarray:
    """Offline optimum: evict the non-selected residents selected again
    farthest in the future (never again first; ties by smaller position)."""
    _check_trace(trace, B)
    T = trace.shape[0]
    nxt = next_use(trace)
    NEVER = T + 1
    nu: Dict[int, int] = {}  # resident position -> its next selection step
    out = np.empty(T, dtype=np.int64)
    for t in range(T):
        sel = [int(p) for p in trace[t]]
        selset = set(sel)
        new = [p for p in sel if p not in nu]
        need = len(new) - (B - len(nu))
        if need > 0:
            # largest next use first; among equals the smaller position
            cand = [(-nu[p], p) for p in nu if p not in selset]
            for _, p in heapq.nsmallest(need, cand):
                del nu[p]
        for p in sel:
            nu[p] = nxt[t].get(p, NEVER)
        out[t] = len(new)
    return out


def simulate(trace: np.ndarray, policy: str, B: int, seed: int = 0) -> np.ndarray:
    """Per-step miss counts of one unit's trace under a policy."""
    if policy == "swap":
        if B != trace.shape[1]:
            raise ValueError("Swap-vanilla keeps exactly the selection: B must equal k")
        return misses_swap(trace)
    if policy == "lru":
        return misses_lru(trace, B)
    if policy == "fifo":
        return misses_fifo(trace, B)
    if policy == "random":
        return misses_random(trace, B, seed)
    if policy == "belady":
        return misses_belady(trace, B)
    raise ValueError(f"unknown policy {policy!r}")


# The page's seven configurations (policy, B as a multiple of k).
STUDY = (("swap", 1), ("lru", 2), ("fifo", 2), ("random", 2), ("belady", 2), ("lru", 4),
         ("belady", 4))


def study(traces: np.ndarray, configs: Sequence = STUDY, skip_cold: bool = True,
          seed: int = 0) -> List[dict]:
    """Mean per-step miss rate of each (policy, B/k) over every unit's trace.

    traces: [steps][units][k]. With skip_cold the first step (empty buffer:
    all k miss under every policy) is left out of the mean."""
    T, n, k = traces.shape
    rows = []
    for policy, mult in configs:
        B = mult * k
        t0 = time.perf_counter()
        per_unit = np.stack([simulate(traces[:, u, :], policy, B, seed + u) for u in range(n)])
        rate = per_unit / float(k)  # [units][steps]
        lo = 1 if skip_cold and T > 1 else 0
        rows.append({"policy": policy, "B": B, "mean_miss_rate": float(rate[:, lo:].mean()),
                     "per_step": rate.mean(axis=0), "seconds": time.perf_counter() - t0})
    return rows


def sweep_B(traces: np.ndarray, policies: Sequence[str] = ("lru", "belady"),
            mults: Sequence[float] = (1.0, 1.25, 1.5, 2.0, 3.0, 4.0), skip_cold: bool = True,
            seed: int = 0) -> List[dict]:
    """Mean per-step miss rate of each policy at B = mult * k (at least k) over
    every unit's trace: the page weighs a larger buffer (fewer misses)
    against its HBM and probe cost."""
    T, n, k = traces.shape
    lo = 1 if skip_cold and T > 1 else 0
    rows = []
    for mult in mults:
        B = max(k, int(round(mult * k)))
        for pol in policies:
            per_unit = np.stack([simulate(traces[:, u, :], pol, B, seed + u) for u in range(n)])
            rate = per_unit / float(k)
            rows.append({"policy": pol, "B": B, "mean_miss_rate": float(rate[:, lo:].mean())})
    return rows


def main() -> None:
    from . import inputs as I

    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--steps", type=int, default=None, help="decode steps (default: the workload's)")
    ap.add_argument("--units", type=int, default=None, help="first N (request, layer) units only")
    ap.add_argument("--sweep", action="store_true",
                    help="LRU and Belady at B = 1, 1.25, 1.5, 2, 3, 4 times k instead of the study")
    args = ap.parse_args()
    w = I.workload(args.workload)
    steps = args.steps or w.steps
    traces = I.gen_traces(w, steps)
    if args.units:
        traces = traces[:, : args.units, :]
    print(f"workload {w.name}: {traces.shape[1]} units x {steps} steps, k = {w.k}; "
          "mean per-step miss rate over steps 1.. (step 0 misses all)")
    if args.sweep:
        print(f"{'policy':8s} {'B':>6s} {'miss rate':>10s}")
        for r in sweep_B(traces):
            print(f"{r['policy']:8s} {r['B']:6d} {r['mean_miss_rate']:10.4f}")
        return
    print(f"{'policy':8s} {'B':>6s} {'miss rate':>10s} {'seconds':>8s}")
    for r in study(traces):
        print(f"{r['policy']:8s} {r['B']:6d} {r['mean_miss_rate']:10.4f} {r['seconds']:8.2f}")


if __name__ == "__main__":
    main()
