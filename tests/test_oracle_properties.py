"""Property-based pins of the oracle's selection and scoring (hypothesis draws
the cases; each is checked against an independent definition).

* Selection (Q-Filters page, "How it works" step 4 and "Metal kernels" tie
  paragraph; L2Norm page, "How it works" step 3): on up to 12 rows drawn from
  a small value set (so that exact ties and signed zeros are common), with
  any budget, sinks and recent window the rules allow, the kept
  rows equal the unique set found by brute-force enumeration.
* Scoring (L2Norm page, "How it works" step 1; Q-Filters page, "How it works"
  step 3): on small integer-valued float32 keys every product and partial sum
  is exact in fp64, so the oracle's score is the exactly rounded float32 of
  the integer norm or dot product, computed here from integers.
"""
import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from tests import refs

VALUES = [-2.0, -1.0, -0.0, 0.0, 0.5, 1.0, 3.0]   # finite: the oracle refuses non-finite scores


@st.composite
def selection_case(draw):
    n = draw(st.integers(0, 12))
    s = draw(st.lists(st.sampled_from(VALUES), min_size=n, max_size=n))
    budget = draw(st.integers(1, 13))
    n_sink = draw(st.integers(0, budget - 1))
    recent = draw(st.integers(0, budget - 1 - n_sink))
    keep = draw(st.sampled_from(["high", "low"]))
    return s, budget, n_sink, recent, keep


@settings(max_examples=400, deadline=None)
@given(selection_case())
def test_selection_equals_brute_force(case):
    s, budget, n_sink, recent, keep = case
    got = oracle.select(np.array(s, dtype=np.float32), budget, n_sink, recent, keep).tolist()
    assert got == refs.brute_force_select(s, budget, n_sink, recent, keep)
    assert len(got) == min(len(s), budget)


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 6).flatmap(lambda n: st.tuples(
    st.lists(st.lists(st.integers(-64, 64), min_size=16, max_size=16), min_size=n, max_size=n),
    st.lists(st.integers(-8, 8), min_size=16, max_size=16), st.sampled_from([1, -1]))))
def test_scores_of_integer_keys_are_exact(case):
    rows, f, sign = case
    k = np.array(rows, dtype=np.float32)
    l2 = oracle.score(k, "l2")
    want_l2 = np.array([np.float32(math.sqrt(sum(x * x for x in r))) for r in rows], dtype=np.float32)
    assert np.array_equal(l2.view(np.int32), want_l2.view(np.int32))
    proj = oracle.score(k, "proj", np.array(f, dtype=np.float32), sign)
    dots = [sign * sum(a * b for a, b in zip(r, f)) for r in rows]
    want_p = np.array([np.float32(d) + np.float32(0.0) for d in dots], dtype=np.float32)   # -0 stored as +0
    assert np.array_equal(proj.view(np.int32), want_p.view(np.int32))
