"""The allocation-free selection (kv_evict_topk_noalloc) against kv_evict_topk
with a caller-allocated workspace, through the C ABI: identical keep_idx on
two calls in a row, the second smaller than the first, both large enough to
need the multi-block selection's scratch; a call that needs no scratch; a
size whose scratch would exceed the static array, rejected before launch; and
the call captured in a HIP graph and replayed on new scores."""
import ctypes

import numpy as np
import pytest

import oracle
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


def _scores(G, n, seed, ties):
    rng = np.random.default_rng(seed)
    if ties:
        return rng.integers(-40, 40, size=(G, n)).astype(np.float32) / 8.0
    return rng.standard_normal((G, n)).astype(np.float32)


def _both(G, n_kept, S, budget, n_sink, recent, keep, seed, ties=False):
    import torch
    from kv_cache_token_amd import api
    sk = torch.from_numpy(_scores(G, budget, seed, ties)).cuda()
    sn = torch.from_numpy(_scores(G, max(S, 1), seed + 1, ties)).cuda()
    shape = api.make_shape(1, 1, G, "bf16")
    p = api.make_params(budget, n_sink, recent, keep)
    need = api.kv_evict_workspace_size(shape, n_kept, S, p)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    ref = torch.full((G, budget), -7, dtype=torch.int32, device="cuda")
    got = torch.full((G, budget), -9, dtype=torch.int32, device="cuda")
    api.kv_evict_topk(sk, sn, shape, n_kept, S, p, ref, ws)
    api.kv_evict_topk_noalloc(sk, sn, shape, n_kept, S, p, got)
    torch.cuda.synchronize()
    n_out = min(n_kept + S, budget)
    ref_h, got_h = ref.cpu().numpy(), got.cpu().numpy()
    assert np.array_equal(ref_h[:, :n_out], got_h[:, :n_out]), "noalloc selection differs from kv_evict_topk"
    # and both equal the oracle's ranking on the first and last group
    for g in (0, G - 1):
        s = np.concatenate([sk[g, :n_kept].cpu().numpy(), sn[g, :S].cpu().numpy()])
        want = oracle.select(s, budget, n_sink, recent, keep)
        assert np.array_equal(got_h[g, :n_out], want.astype(np.int32)), "group %d differs from the oracle" % g
    return need


def test_noalloc_matches_workspace_selection_on_two_calls():
    say("noalloc: call 1 (G 6, 300000 rows)")
    need1 = _both(6, 150000, 150000, 150000, 4, 16, "low", 11)
    say("noalloc: call 2 (G 3, 270000 rows, ties)")
    need2 = _both(3, 100000, 170000, 100000, 4, 0, "high", 12, ties=True)
    assert need1 > need2 > 0
    say("noalloc: call 3 (on chip, no scratch)")
    assert _both(5, 4096, 4096, 4096, 4, 0, "low", 13) == 0


def test_noalloc_rejects_sizes_beyond_the_scratch_before_launch():
    from kv_cache_token_amd import _lib, api
    shape = api.make_shape(1, 1, 4000, "bf16")
    p = api.make_params(1 << 21, 4, 0, "low")
    assert api.kv_evict_workspace_size(shape, 1 << 21, 1 << 21, p) > _lib.KVX_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: the size check comes first
    rc = _lib.lib().kv_evict_topk_noalloc(fake, fake, shape, 1 << 21, 1 << 21, p, fake, None)
    assert rc == _lib.KVX_ERANGE
    assert b"scratch" in _lib.lib().kvx_last_error()


def test_noalloc_selection_inside_a_captured_graph():
    """The use the entry point is for: a selection that needs the multi-block
    scratch, captured in a HIP graph (nothing allocated during capture) and
    replayed on new scores written between replays, each replay equal to
    kv_evict_topk with a caller-allocated workspace."""
    import torch
    from kv_cache_token_amd import api
    G, n_kept, S, budget = 4, 140000, 140000, 140000
    shape, p = api.make_shape(1, 1, G, "bf16"), api.make_params(budget, 4, 8, "low")
    need = api.kv_evict_workspace_size(shape, n_kept, S, p)
    assert need > 0
    sk = torch.empty((G, budget), device="cuda")
    sn = torch.empty((G, S), device="cuda")
    got = torch.empty((G, budget), dtype=torch.int32, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(got)
    stream = torch.cuda.Stream()
    sk.copy_(torch.from_numpy(_scores(G, budget, 40, False)))
    sn.copy_(torch.from_numpy(_scores(G, S, 41, False)))
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):     # first call outside capture: the scratch address is looked up
        api.kv_evict_topk_noalloc(sk, sn, shape, n_kept, S, p, got, stream=stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        api.kv_evict_topk_noalloc(sk, sn, shape, n_kept, S, p, got, stream=stream)
    torch.cuda.synchronize()
    for rep in range(3):
        sk.copy_(torch.from_numpy(_scores(G, budget, 50 + rep, rep == 1)))
        sn.copy_(torch.from_numpy(_scores(G, S, 60 + rep, rep == 1)))
        got.fill_(-5)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        api.kv_evict_topk(sk, sn, shape, n_kept, S, p, ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "replay %d" % rep
