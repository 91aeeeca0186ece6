"""Independent brute-force models used to pin the oracle's RESOLVE.

Nothing here imports the oracle. The LRU model keeps an explicit recency list
of resident logical positions (most recent first) and no stamps at all; slot
ids are assigned in a second, separate pass. It is written from the same rules
the HiSparse summary page (marsggbo.github.io, 2026-09-23) gives in sections
3-5: hits are kept and become most recent, fetched misses rank right after the
hits, the least recently used non-selected residents are evicted, nothing is
evicted while a slot is still free; plus the tie rule that equally recent
positions leave in ascending logical position.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Set, Tuple


class BruteLRU:
    """Recency-list LRU over set requests."""

    def __init__(self, B: int):
        self.B = B
        self.order: List[int] = []  # resident positions, most recent first
        self.slot_of: Dict[int, int] = {}
        self.free: List[int] = list(range(B))  # never-used slots, ascending

    def resident(self) -> Set[int]:
        return set(self.order)

    def grow(self, new_B: int) -> None:
        """More capacity: the added slots are free (never used), after the
        existing ones."""
        assert new_B >= self.B
        self.free.extend(range(self.B, new_B))
        self.B = new_B

    def step(self, sel: Sequence[int]) -> Tuple[List[int], int, List[int]]:
        """Returns (slots aligned with sel, miss count, evicted positions)."""
        S = set(sel)
        res = set(self.order)
        hits = [p for p in sel if p in res]
        misses = [p for p in sel if p not in res]
        need = len(res) + len(misses) - self.B
        evicted: List[int] = []
        if need > 0:
            # walk from the least recent end, skipping selected positions
            for p in reversed(self.order):
                if len(evicted) == need:
                    break
                if p not in S:
                    evicted.append(p)
        ev = set(evicted)
        survivors = [p for p in self.order if p not in S and p not in ev]
        # within one step's group, the larger position counts as more recent,
        # so the smaller one is evicted first among equals
        self.order = sorted(hits, reverse=True) + sorted(misses, reverse=True) + survivors
        # slot pass: free slots first (ascending), then the evicted positions'
        # slots; all victim slots sorted ascending, paired with misses in
        # selection order
        n_free_used = min(len(misses), len(self.free))
        vslots = self.free[:n_free_used] + [self.slot_of[p] for p in evicted]
        self.free = self.free[n_free_used:]
        for p in evicted:
            del self.slot_of[p]
        vslots.sort()
        for p, s in zip(misses, vslots):
            self.slot_of[p] = s
        return [self.slot_of[p] for p in sel], len(misses), evicted


def belady_misses(trace: Sequence[Sequence[int]], B: int) -> int:
    """Offline MIN over set requests: on each miss that needs room, evict the
    non-selected resident whose next use lies farthest in the future (never
    used again counts as infinitely far; ties go to the smaller position)."""
    T = len(trace)
    next_use: List[Dict[int, int]] = [dict() for _ in range(T)]
    last: Dict[int, int] = {}
    for t in range(T - 1, -1, -1):
        next_use[t] = dict(last)  # next use strictly after t
        for p in trace[t]:
            last[p] = t
    res: Set[int] = set()
    total = 0
    INF = 1 << 60
    for t, sel in enumerate(trace):
        S = set(sel)
        misses = [p for p in sel if p not in res]
        total += len(misses)
        need = len(res) + len(misses) - B
        if need > 0:
            cands = [p for p in res if p not in S]
            cands.sort(key=lambda p: (-next_use[t].get(p, INF), p))
            for p in cands[:need]:
                res.discard(p)
        res |= S
    return total


def lru_misses(trace: Sequence[Sequence[int]], B: int) -> List[int]:
    m = BruteLRU(B)
    return [m.step(list(sel))[1] for sel in trace]


def check_invariants(before_pos, after_pos, after_stamp, clock_after, topk, slots, miss,
                     B: int, seen: Set[int]) -> None:
    """State invariants after one successful resolve (raise AssertionError).

    before_pos/after_pos: slot -> position arrays (-1 empty); seen: every
    position selected so far, this step included."""
    import numpy as np

    before_pos = np.asarray(before_pos)
    after_pos = np.asarray(after_pos)
    after_stamp = np.asarray(after_stamp, dtype=np.int64)
    topk = [int(x) for x in topk]
    slots = [int(x) for x in slots]
    T = set(topk)
    prior = set(int(p) for p in before_pos if p >= 0)
    occ = [int(p) for p in after_pos if p >= 0]
    # every selected position is resident, and the slot vector is aligned
    for p, s in zip(topk, slots):
        assert 0 <= s < B and int(after_pos[s]) == p
    # the page table is injective on occupied slots
    assert len(occ) == len(set(occ))
    # the misses are exactly the selected positions not resident before
    assert miss == len(T - prior)
    after = set(occ)
    assert after - prior == T - prior
    # evicted positions were resident before and not selected
    evicted = prior - after
    assert evicted <= prior - T
    # nothing is evicted while free slots remain
    assert len(occ) == min(B, len(seen))
    # recency stamps
    c = int(clock_after)
    for s in range(B):
        p = int(after_pos[s])
        if p in T:
            want = 2 * c if p in prior else 2 * c - 1
            assert after_stamp[s] == want
        else:
            assert after_stamp[s] < 2 * c - 1
