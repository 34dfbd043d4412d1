"""Prepared block streams (EvictingCache.plan) keep every buffer their calls
point at alive and leave the cache's state consistent.

* A stream whose selections run over more than 262144 rows per group needs the
  multi-block selection's workspace, and its second evicting call needs a
  larger one than its first (19 then 22 row blocks of 16384).  The plan must
  hold on to the first workspace after the cache replaced it: memory allocated
  after planning must not be written by the replay, and the replay must equal
  the eager run and the oracle (its rules on the GPU's scores) bit for bit.
* A key-SVD fallback cache leaves planning with no filters (nothing has run);
  after a run it points at the filters the run froze.
"""
import numpy as np
import pytest

import oracle
from kv_cache_token_amd import synth
from tests.gpu_util import assert_states_equal, gpu_state_arrays, host_rows, say

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


def _blocks(G, sizes, seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = []
    for S in sizes:
        k = torch.randn((G, S, D), generator=gen, device="cuda").to(torch.bfloat16)
        v = torch.randn((G, S, D), generator=gen, device="cuda").to(torch.bfloat16)
        out.append((k, v))
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("keep", ["low", "high"])
def test_plan_keeps_a_replaced_workspace_alive(keep):
    import torch
    from kv_cache_token_amd import api
    from kv_cache_token_amd.cache import EvictingCache
    L, B, H, budget, S = 1, 1, 2, 200000, 150000
    G = L * B * H
    blocks = _blocks(G, (S, S, S), 4242)
    params = api.make_params(budget, 4, 0, keep)
    shape = api.make_shape(L, B, H, "bf16")
    ws1 = api.kv_evict_workspace_size(shape, S, S, params)
    ws2 = api.kv_evict_workspace_size(shape, budget, S, params)
    assert 0 < ws1 < ws2, (ws1, ws2)

    say("plan: eager run with the oracle in lockstep (%s)" % keep)
    eager = EvictingCache(L, B, H, budget, 4, 0, keep, "l2")
    lock = oracle.OracleCache(G, D, "bf16", budget, 4, 0, keep, "l2")
    groups = list(range(G))
    for k, v in blocks:
        eager.update(k, v)
        s = host_rows(eager.last_scores(), groups, "f32")
        lock.update(host_rows(k, groups, "bf16"), host_rows(v, groups, "bf16"), scores_in=s)
    torch.cuda.synchronize()
    want = gpu_state_arrays(eager, groups)
    assert_states_equal(want, lock, groups, "eager")

    say("plan: replay after the first workspace was replaced")
    c = EvictingCache(L, B, H, budget, 4, 0, keep, "l2")
    plan = c.plan(blocks)
    assert plan.names.count("kv_evict_topk") == 2
    # allocations made after planning: none may be one the replay writes into
    probes = [torch.full((ws1,), 0xA5, dtype=torch.uint8, device="cuda") for _ in range(64)]
    for rep in range(2):
        for x in c.buffers():
            x.view(torch.uint8).fill_(0x3C)
        plan.run()
        torch.cuda.synchronize()
        for p in probes:
            assert bool((p == 0xA5).all()), "the replay wrote into memory allocated after planning"
        got = gpu_state_arrays(c, groups)
        assert_states_equal(got, lock, groups, "replay %d" % rep)
    assert c.n_kept == budget and c.offset == 3 * S


def test_fallback_plan_points_at_its_filters_only_after_a_run():
    import torch
    from kv_cache_token_amd.cache import EvictingCache
    G = 8
    rng = np.random.default_rng(3)
    mu = rng.standard_normal(D)
    mu /= np.linalg.norm(mu)
    K = (rng.uniform(0.5, 2.0, (G, 400, 1)) * mu + 0.5 * rng.standard_normal((G, 400, D))).astype(np.float32)
    kt = synth.host_to_torch(synth.encode(K, "bf16"), "bf16").cuda()
    blocks = [(kt[:, :100].contiguous(), kt[:, :100].contiguous()),
              (kt[:, 100:].contiguous(), kt[:, 100:].contiguous())]
    eager = EvictingCache(2, 1, 4, 64, 4, 0, mode="proj", calib_tokens=128)
    for k, v in blocks:
        eager.update(k, v)
    c = EvictingCache(2, 1, 4, 64, 4, 0, mode="proj", calib_tokens=128)
    plan = c.plan(blocks)
    assert c.filters is None and c.calibrating and c.n_kept == 0 and c.calib_status is None
    k0, v0, s0, p0 = c.kept()
    assert k0.shape[1] == 0 and s0 is None
    plan.run()
    plan.check()
    assert not c.calibrating and c.n_kept == 64 and c.offset == 400
    assert torch.equal(c.filters, eager.filters)
    for x, y in zip(c.kept(), eager.kept()):
        assert torch.equal(x, y)
