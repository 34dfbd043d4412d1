"""Independent reference implementations used to pin the oracle.

None of these share code with ``oracle/``; each one reaches the selection rule a
different way, so that a slip in the oracle (a dropped term, a reversed tie,
a wrong protected window) fails at least one of them.
"""
from __future__ import annotations

import heapq
import itertools
from typing import Callable, Iterable, List, Sequence

import numpy as np


def protected_rows(n_total: int, n_sink: int, recent: int) -> set:
    return set(range(min(n_sink, n_total))) | set(range(max(0, n_total - recent), n_total))


def beats(s: Sequence[float], a: int, b: int, keep: str) -> bool:
    """True if row a ranks strictly ahead of row b: better score, or equal score and lower row."""
    if s[a] == s[b]:
        return a < b
    return s[a] > s[b] if keep == "high" else s[a] < s[b]


def brute_force_select(s: Sequence[float], budget: int, n_sink: int, recent: int, keep: str) -> List[int]:
    """Enumerate every candidate kept set of the right size that contains the
    protected rows, and return the one (it must be unique) in which every kept
    unprotected row beats every evicted row.  Tiny n only."""
    n = len(s)
    if n <= budget:
        return list(range(n))
    P = protected_rows(n, n_sink, recent)
    free = [r for r in range(n) if r not in P]
    take = budget - len(P)
    valid = []
    for comb in itertools.combinations(free, take):
        kept = set(comb)
        evicted = [r for r in free if r not in kept]
        if all(beats(s, a, b, keep) for a in kept for b in evicted):
            valid.append(sorted(P | kept))
    assert len(valid) == 1, "the kept set must be unique under the (score, row) order"
    return valid[0]


def lexsort_select(s: np.ndarray, budget: int, n_sink: int, recent: int, keep: str) -> np.ndarray:
    """numpy lexsort ranking of the unprotected rows (primary score, secondary row)."""
    s = np.asarray(s, dtype=np.float64)
    n = s.size
    if n <= budget:
        return np.arange(n)
    P = protected_rows(n, n_sink, recent)
    free = np.array([r for r in range(n) if r not in P], dtype=np.int64)
    primary = -s[free] if keep == "high" else s[free]
    order = np.lexsort((free, primary))
    kept = set(free[order[:budget - len(P)]].tolist()) | P
    return np.array(sorted(kept), dtype=np.int64)


def heap_stream(scores_by_pos: Sequence[float], budget: int, n_sink: int, keep: str) -> List[int]:
    """Classic streaming keep-k-best with a heap (recent = 0): the first n_sink
    positions are kept unconditionally; every later token enters a bounded
    min-heap keyed so that the worst element sits on top and is popped when the
    heap exceeds budget - n_sink.  Returns the kept positions, ascending."""
    sinks, heap = [], []
    cap = budget - n_sink
    for p, s in enumerate(scores_by_pos):
        if p < n_sink:
            sinks.append(p)
            continue
        # heap top = worst: lowest score (keep-high) / highest score (keep-low);
        # among equal scores the latest position is the worst.
        key = (s if keep == "high" else -s, -p)
        heapq.heappush(heap, (key, p))
        if len(heap) > cap:
            heapq.heappop(heap)
    return sorted(sinks + [p for _, p in heap])


def decode_rule(state_s: List[float], state_pos: List[int], new_s: float, new_pos: int,
                budget: int, n_sink: int, recent: int, keep: str):
    """Single-token eviction written as 'drop the worst candidate, shift the rest':
    the candidate rows are those outside the sinks and the recent window of the
    concatenation; the worst is the lowest-ranked (for equal scores the later
    row).  Returns the new (scores, positions)."""
    s = list(state_s) + [new_s]
    pos = list(state_pos) + [new_pos]
    n = len(s)
    if n <= budget:
        return s, pos
    cands = [r for r in range(n) if r >= n_sink and r < n - recent]
    worst = cands[0]
    for r in cands[1:]:
        if not beats(s, r, worst, keep):   # r ranks behind (or is later on a tie)
            worst = r
    del s[worst]
    del pos[worst]
    return s, pos


SelectFn = Callable[[np.ndarray, int, int, int, str], np.ndarray]


def selection_cases(seed: int = 0) -> Iterable:
    """Small cases with many exact ties, both keep directions, assorted protection."""
    rng = np.random.default_rng(seed)
    for n in range(1, 12):
        for budget in range(1, n + 2):
            for n_sink in range(0, 3):
                for recent in range(0, 3):
                    if n_sink + recent >= budget:
                        continue
                    for keep in ("high", "low"):
                        s = rng.integers(-2, 3, size=n).astype(np.float32)
                        yield s, budget, n_sink, recent, keep


def check_selection(select: SelectFn, n_cases: int = 10 ** 9, seed: int = 0) -> None:
    """Every pin on the selection rule at once; raises AssertionError on the first miss."""
    for i, (s, budget, n_sink, recent, keep) in enumerate(selection_cases(seed)):
        if i >= n_cases:
            break
        got = np.asarray(select(s, budget, n_sink, recent, keep)).tolist()
        want = brute_force_select(s.tolist(), budget, n_sink, recent, keep)
        assert got == want, (s.tolist(), budget, n_sink, recent, keep, got, want)
    # all-equal scores: exactly the lowest unprotected rows survive besides the protected
    s = np.full(40, 1.5, dtype=np.float32)
    got = np.asarray(select(s, 10, 2, 3, "high")).tolist()
    assert got == [0, 1, 2, 3, 4, 5, 6, 37, 38, 39], got
    got = np.asarray(select(s, 10, 2, 3, "low")).tolist()
    assert got == [0, 1, 2, 3, 4, 5, 6, 37, 38, 39], got
    # sinks and the recent window survive even with the worst possible scores
    s = np.arange(30, dtype=np.float32)
    got = np.asarray(select(s, 8, 2, 2, "high")).tolist()
    assert got == [0, 1, 24, 25, 26, 27, 28, 29], got
    got = np.asarray(select(s, 8, 2, 2, "low")).tolist()
    assert got == [0, 1, 2, 3, 4, 5, 28, 29], got
    got = np.asarray(select(s[::-1].copy(), 8, 2, 2, "low")).tolist()
    assert got == [0, 1, 24, 25, 26, 27, 28, 29], got
