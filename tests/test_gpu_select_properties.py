"""Property-based parity of the selection (kv_evict_topk, and the allocation-
free kv_evict_topk_noalloc) with the oracle on drawn cases: group counts,
budgets from 1 to 300000, kept and incoming row counts on both sides of every
on-chip bound (register-held keys up to 32768 rows, streamed keys up to
262144, the multi-block selection beyond), sinks and recent windows, both
directions, and score distributions with heavy exact ties, signed zeros or a
single value.  keep_idx must equal the oracle's selection, row for row.
Hypothesis runs derandomised, so every failure names a reproducible case."""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
BOUNDS = [1, 2, 1024, 4096, 32768, 32769, 262144, 262145, 300000]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


@st.composite
def case(draw):
    budget = draw(st.one_of(st.integers(1, 5000), st.sampled_from([4096, 32768, 150000])))
    n_kept = draw(st.integers(0, budget))
    near = draw(st.sampled_from(BOUNDS))
    n_total = max(n_kept, min(near + draw(st.integers(-3, 3)), n_kept + 300000))
    S = max(0, n_total - n_kept)
    n_sink = draw(st.integers(0, min(8, budget - 1)))
    recent = draw(st.integers(0, budget - 1 - n_sink)) if draw(st.booleans()) else 0
    keep = draw(st.sampled_from(["high", "low"]))
    dist = draw(st.sampled_from(["gauss", "ties", "zeros", "constant"]))
    G = draw(st.integers(1, 3))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return G, budget, n_kept, S, n_sink, recent, keep, dist, seed


def _scores(rng, G, n, dist):
    if dist == "gauss":
        return rng.standard_normal((G, n)).astype(np.float32)
    if dist == "ties":
        return (rng.integers(-6, 6, size=(G, n)) / 4.0).astype(np.float32)
    if dist == "zeros":
        return np.where(rng.random((G, n)) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    return np.full((G, n), 1.5, dtype=np.float32)


@settings(max_examples=120, deadline=None, derandomize=True)
@given(case())
def test_selection_matches_the_oracle(c):
    import torch
    from kv_cache_token_amd import api
    G, budget, n_kept, S, n_sink, recent, keep, dist, seed = c
    rng = np.random.default_rng(seed)
    s = _scores(rng, G, n_kept + S, dist)
    say("select case G=%d budget=%d n_kept=%d S=%d sink=%d recent=%d %s %s" % (G, budget, n_kept, S, n_sink,
                                                                            recent, keep, dist))
    sk = torch.zeros((G, budget), device="cuda")
    sk[:, :n_kept] = torch.from_numpy(s[:, :n_kept]).cuda()
    sn = torch.from_numpy(np.ascontiguousarray(s[:, n_kept:])).cuda() if S else torch.zeros((G, 1), device="cuda")
    shape, params = api.make_shape(1, 1, G, "bf16"), api.make_params(budget, n_sink, recent, keep)
    need = api.kv_evict_workspace_size(shape, n_kept, S, params)
    ws = torch.full((max(need, 1),), 0x77, dtype=torch.uint8, device="cuda")
    a = torch.full((G, budget), -1, dtype=torch.int32, device="cuda")
    b = torch.full((G, budget), -1, dtype=torch.int32, device="cuda")
    api.kv_evict_topk(sk, sn, shape, n_kept, S, params, a, ws if need else None)
    api.kv_evict_topk_noalloc(sk, sn, shape, n_kept, S, params, b)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    n_out = min(n_kept + S, budget)
    for g in range(G):
        want = oracle.select(s[g], budget, n_sink, recent, keep)
        assert np.array_equal(a[g, :n_out], want), "group %d (workspace)" % g
        assert np.array_equal(b[g, :n_out], want), "group %d (no allocation)" % g
        assert (a[g, n_out:] == -1).all() and (b[g, n_out:] == -1).all()
