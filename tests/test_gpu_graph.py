"""A captured HIP graph of a planned block stream replays to the same bytes as
eager execution, replay after replay, with unrelated eager work and
synchronisations in between (the library records no memset nodes)."""
import numpy as np
import pytest

from kv_cache_token_amd import synth

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _snapshot(cache):
    import torch
    k, v, s, p = cache.kept()
    return [k.view(torch.int16).cpu(), v.view(torch.int16).cpu(), s.cpu(), p.cpu()]


@pytest.mark.parametrize("mode,keep,sign", [("l2", "low", 1), ("proj", "high", -1)])
def test_graph_replays_match_eager(mode, keep, sign):
    import torch
    from kv_cache_token_amd.cache import EvictingCache
    G, budget = 24, 300
    rng = np.random.default_rng(5)
    f = torch.from_numpy(rng.standard_normal((2, 12, D)).astype(np.float32)).cuda()
    stream = torch.cuda.Stream()
    blocks = []
    for c, S in enumerate((256, 256, 100, 512)):
        k = synth.host_to_torch(synth.custom_keys((G, S, D), 40 + c, "bf16"), "bf16").cuda()
        v = synth.host_to_torch(synth.custom_keys((G, S, D), 50 + c, "bf16"), "bf16").cuda()
        blocks.append((k, v))
    cache = EvictingCache(2, 1, 12, budget, 4, 16, keep, mode, f if mode == "proj" else None, sign, stream=stream)
    plan = cache.plan(blocks)
    with torch.cuda.stream(stream):
        plan.run()
    torch.cuda.synchronize()
    eager = _snapshot(cache)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        plan.run()
    torch.cuda.synchronize()
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(4):
        for bufset in cache._bufs:           # scribble over the state so that a replay must rebuild it
            for buf in bufset:
                buf.view(torch.uint8).fill_(0x5A)
        cache.keep_idx.fill_(-3)
        junk.add_(1.0).sum().item()          # unrelated eager work and a synchronisation
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(cache)
        for a, b in zip(eager, got):
            assert torch.equal(a, b), "replay %d differs from eager" % rep
