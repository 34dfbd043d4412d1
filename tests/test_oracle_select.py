"""Pins for the oracle's selection rule (protected top-k with lower-row ties).

Rule (Q-Filters page, "How it works" step 4 and "Metal kernels" tie paragraph;
L2Norm page, "How it works" step 3): when over budget, keep the protected rows
(first n_sink, last `recent`) plus the best remaining rows, ties to the lower
row, in row order.  Pinned against brute-force enumeration, numpy lexsort and
the tie / protection cases the pages describe, and the pins are shown to catch
plausible mistakes (mutants).
"""
import numpy as np
import pytest

import oracle
from tests import refs


def oracle_select(s, budget, n_sink, recent, keep):
    return oracle.select(s, budget, n_sink, recent, keep)


def test_oracle_select_matches_brute_force_and_tie_cases():
    refs.check_selection(oracle_select)


@pytest.mark.parametrize("keep", ["high", "low"])
@pytest.mark.parametrize("n,budget,n_sink,recent", [(1000, 300, 4, 0), (513, 512, 4, 0),
                                                    (2049, 2048, 4, 512), (777, 100, 0, 99)])
def test_oracle_select_matches_lexsort(keep, n, budget, n_sink, recent):
    rng = np.random.default_rng(n + budget)
    s = rng.standard_normal(n).astype(np.float32)
    s[rng.integers(0, n, size=n // 5)] = 0.25          # planted exact ties
    got = oracle.select(s, budget, n_sink, recent, keep)
    want = refs.lexsort_select(s, budget, n_sink, recent, keep)
    assert np.array_equal(got, want)
    assert got.size == min(n, budget)


def test_under_and_at_budget_keep_everything():
    s = np.arange(5, dtype=np.float32)
    assert oracle.select(s, 5, 1, 1, "high").tolist() == [0, 1, 2, 3, 4]
    assert oracle.select(s, 9, 1, 1, "low").tolist() == [0, 1, 2, 3, 4]
    assert oracle.select(s[:0], 4, 1, 1, "low").tolist() == []


def test_signed_zeros_tie_and_lower_row_wins():
    s = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    assert oracle.select(s, 2, 0, 0, "high").tolist() == [0, 1]
    assert oracle.select(s, 2, 0, 0, "low").tolist() == [0, 1]
    s = np.array([1.0, 0.0, -0.0], dtype=np.float32)
    assert oracle.select(s, 2, 0, 0, "low").tolist() == [1, 2]


def test_invalid_parameters_raise():
    s = np.zeros(10, dtype=np.float32)
    for budget, n_sink, recent in [(4, 2, 2), (4, 4, 0), (0, 0, 0), (3, -1, 0)]:
        with pytest.raises(oracle.OracleError):
            oracle.select(s, budget, n_sink, recent, "high")
    with pytest.raises(oracle.OracleError):
        oracle.select(np.array([1.0, np.inf, 0.0], dtype=np.float32), 1, 0, 0, "high")


# --- the pins catch plausible mistakes ------------------------------------

def _mutant_upper_row_ties(s, budget, n_sink, recent, keep):
    n = len(s)
    if n <= budget:
        return np.arange(n)
    P = refs.protected_rows(n, n_sink, recent)
    free = [r for r in range(n) if r not in P]
    key = (lambda r: (-s[r], -r)) if keep == "high" else (lambda r: (s[r], -r))
    return np.array(sorted(P | set(sorted(free, key=key)[:budget - len(P)])))


def _mutant_no_recent(s, budget, n_sink, recent, keep):
    return refs.lexsort_select(s, budget, n_sink, 0, keep) if len(s) > budget else np.arange(len(s))


def _mutant_keep_direction(s, budget, n_sink, recent, keep):
    return refs.lexsort_select(s, budget, n_sink, recent, "low" if keep == "high" else "high")


def _mutant_at_budget_evicts(s, budget, n_sink, recent, keep):
    if len(s) == budget and budget > n_sink + recent:
        return refs.lexsort_select(s, budget - 1, n_sink, recent, keep)
    return refs.lexsort_select(s, budget, n_sink, recent, keep)


def _mutant_budget_excludes_sinks(s, budget, n_sink, recent, keep):
    n = len(s)
    if n <= budget:
        return np.arange(n)
    P = refs.protected_rows(n, n_sink, recent)
    free = np.array([r for r in range(n) if r not in P])
    prim = -np.asarray(s)[free] if keep == "high" else np.asarray(s)[free]
    order = np.lexsort((free, prim))
    return np.array(sorted(set(free[order[:budget - recent]].tolist()) | P))


@pytest.mark.parametrize("mutant", [_mutant_upper_row_ties, _mutant_no_recent, _mutant_keep_direction,
                                    _mutant_at_budget_evicts, _mutant_budget_excludes_sinks])
def test_selection_pins_reject_mutants(mutant):
    with pytest.raises(AssertionError):
        refs.check_selection(mutant)
