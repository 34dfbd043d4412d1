"""Randomised streams through the whole cache, in lockstep with the oracle.

Each case draws a configuration (element type, head dim, groups, budget,
sinks, recent window, direction, scorer, sign) and a stream of blocks of
random sizes -- single tokens, blocks that fill the cache exactly, blocks far
larger than the budget, heavy score ties -- and checks after every block that
the GPU's kept rows, K/V bytes, stored scores and positions equal what the
oracle's rules give on the GPU's scores, and that the GPU's scores lie within
the tolerance of the oracle's.  The draws are seeded, so every case is
reproducible by its id."""
import numpy as np
import pytest

import oracle
from kv_cache_token_amd import synth
from tests.gpu_util import assert_scores_close, assert_states_equal, gpu_state_arrays, host_rows, \
    oracle_scores, score_scales

pytestmark = pytest.mark.gpu
N_CASES = 500


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


def _case(seed):
    rng = np.random.default_rng([4242, seed])
    dtype = str(rng.choice(["bf16", "f16", "f32"]))
    Dd = int(rng.choice([64, 128, 256]))
    L, B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 5))
    budget = int(rng.choice([2, 3, 8, 64, 257, 1000, 4096]))
    n_sink = int(rng.integers(0, min(5, budget)))
    recent = int(rng.integers(0, budget - n_sink)) if rng.random() < 0.5 else 0
    mode = str(rng.choice(["l2", "proj"]))
    keep = "high" if mode == "proj" else str(rng.choice(["low", "high"]))
    sign = int(rng.choice([1, -1]))
    sizes = []
    for _ in range(int(rng.integers(2, 7))):
        kind = rng.random()
        if kind < 0.3:
            sizes.append(1)
        elif kind < 0.45:
            sizes.append(budget)
        elif kind < 0.6:
            sizes.append(int(rng.integers(budget, 3 * budget + 2)))
        else:
            sizes.append(int(rng.integers(1, budget + 2)))
    ties = bool(rng.random() < 0.3)
    return dict(dtype=dtype, D=Dd, L=L, B=B, H=H, budget=budget, n_sink=n_sink, recent=recent, mode=mode, keep=keep,
                sign=sign, sizes=sizes, ties=ties)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_stream_lockstep_with_oracle(seed):
    import torch
    from kv_cache_token_amd.cache import EvictingCache
    c = _case(seed)
    G, Dd, dt = c["L"] * c["B"] * c["H"], c["D"], c["dtype"]
    rng = np.random.default_rng([4343, seed])
    f_lh = rng.standard_normal((c["L"], c["H"], Dd)).astype(np.float32) if c["mode"] == "proj" else None
    cache = EvictingCache(c["L"], c["B"], c["H"], c["budget"], c["n_sink"], c["recent"], c["keep"], c["mode"],
                          None if f_lh is None else torch.from_numpy(f_lh), c["sign"], dt, head_dim=Dd)
    f_g = None if f_lh is None else np.stack([f_lh[g // (c["B"] * c["H"]), g % c["H"]] for g in range(G)])
    lock = oracle.OracleCache(G, Dd, dt, c["budget"], c["n_sink"], c["recent"], c["keep"], c["mode"], f_g, c["sign"])
    groups = list(range(G))
    for b, S in enumerate(c["sizes"]):
        kind = "dup" if c["ties"] else "gauss"
        K = synth.custom_keys((G, S, Dd), 7000 + 100 * seed + b, dt, kind=kind)
        V = synth.custom_keys((G, S, Dd), 8000 + 100 * seed + b, dt)
        cache.update(synth.host_to_torch(K, dt).cuda(), synth.host_to_torch(V, dt).cuda())
        s_gpu = host_rows(cache.last_scores()[:, :S], groups, "f32")
        lock.update(K, V, scores_in=s_gpu)
        s_ref = oracle_scores(K, dt, c["mode"], f_g, c["sign"])
        assert_scores_close(s_gpu, s_ref, score_scales(K, dt, c["mode"], s_ref, f_g), "case %d block %d" % (seed, b))
        torch.cuda.synchronize()
        assert_states_equal(gpu_state_arrays(cache, groups), lock, groups, "case %d %s block %d" % (seed, c, b))
    assert cache.offset == sum(c["sizes"]) and cache.n_kept == min(sum(c["sizes"]), c["budget"])
