"""The largest sizes the library accepts: a budget of KVX_MAX_BUDGET (2^21
rows) and a concatenation of KVX_MAX_TOTAL (2^22 rows) per group, through the
selection with a caller's workspace and the allocation-free one, and through a
whole evicting call of the cache (multi-block selection, then compaction),
each compared with the oracle, and decode steps that shift a whole 2^21-row
cache in place; one row more is refused before launch."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_states_equal, gpu_state_arrays, host_rows, say

pytestmark = pytest.mark.gpu
D = 128
MAX_BUDGET, MAX_TOTAL = 1 << 21, 1 << 22


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dist", ["gauss", "ties"])
def test_selection_at_the_largest_sizes(dist):
    import torch
    from kv_cache_token_amd import _lib, api
    assert (_lib.KVX_MAX_BUDGET, _lib.KVX_MAX_TOTAL) == (MAX_BUDGET, MAX_TOTAL)
    G, n_kept, S, budget, n_sink, recent = 2, MAX_BUDGET, MAX_TOTAL - MAX_BUDGET, MAX_BUDGET, 4, 1000
    say("selection at %d rows, budget %d (%s)" % (n_kept + S, budget, dist))
    rng = np.random.default_rng(31 if dist == "gauss" else 32)
    if dist == "gauss":
        s = rng.standard_normal((G, n_kept + S)).astype(np.float32)
    else:
        s = (rng.integers(-20, 20, size=(G, n_kept + S)) / 2.0).astype(np.float32)
    sk = torch.from_numpy(np.ascontiguousarray(s[:, :n_kept])).cuda()
    sn = torch.from_numpy(np.ascontiguousarray(s[:, n_kept:])).cuda()
    shape, params = api.make_shape(1, 1, G, "bf16"), api.make_params(budget, n_sink, recent, "high")
    need = api.kv_evict_workspace_size(shape, n_kept, S, params)
    assert need == G * (260 + 2 * 256) * 4                     # 256 row blocks of 16384
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    a = torch.full((G, budget), -1, dtype=torch.int32, device="cuda")
    b = torch.full((G, budget), -2, dtype=torch.int32, device="cuda")
    api.kv_evict_topk(sk, sn, shape, n_kept, S, params, a, ws)
    api.kv_evict_topk_noalloc(sk, sn, shape, n_kept, S, params, b)
    torch.cuda.synchronize()
    a, b = a.cpu().numpy(), b.cpu().numpy()
    for g in range(G):
        want = oracle.select(s[g], budget, n_sink, recent, "high").astype(np.int32)
        assert np.array_equal(a[g], want), "group %d (workspace)" % g
        assert np.array_equal(b[g], want), "group %d (no allocation)" % g
    # one row more: the library refuses it before anything is launched (the
    # buffers are not read; their sizes are the caller's to guarantee)
    rc = _lib.lib().kv_evict_topk(sk.data_ptr(), sn.data_ptr(), shape, n_kept, S + 1, params, ws.data_ptr(),
                                  ws.data_ptr(), need, None)
    assert rc == _lib.KVX_ERANGE and b"KVX_MAX_TOTAL" in _lib.lib().kvx_last_error()


@pytest.mark.timeout(600)
def test_evicting_call_at_the_largest_budget():
    import torch
    from kv_cache_token_amd.cache import EvictingCache
    budget, n_sink, recent = MAX_BUDGET, 4, 512
    say("cache call at budget %d" % budget)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    blocks = []
    for _ in range(2):
        k = torch.randn((1, MAX_BUDGET, D), generator=gen, device="cuda").to(torch.bfloat16)
        v = torch.randn((1, MAX_BUDGET, D), generator=gen, device="cuda").to(torch.bfloat16)
        blocks.append((k, v))
    c = EvictingCache(1, 1, 1, budget, n_sink, recent, "low", "l2")
    lock = oracle.OracleCache(1, D, "bf16", budget, n_sink, recent, "low", "l2")
    for k, v in blocks:
        c.update(k, v)
        s_gpu = host_rows(c.last_scores(), [0], "f32")
        lock.update(host_rows(k, [0], "bf16"), host_rows(v, [0], "bf16"), scores_in=s_gpu)
    torch.cuda.synchronize()
    assert c.n_kept == budget and c.offset == 2 * MAX_BUDGET
    assert_states_equal(gpu_state_arrays(c, [0]), lock, [0], "budget 2^21")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype,Dd", [("bf16", 128), ("f32", 256)])
def test_decode_at_the_largest_budget(dtype, Dd):
    """Single-token calls on a full cache of KVX_MAX_BUDGET rows: each drops
    one row and shifts up to 2^21 rows down in place (a victim near the front
    is planted so that almost the whole cache moves), in lockstep with the
    oracle after every token.  With float32 rows of 256 elements a group's K
    rows span 2 GiB, the most one of the shift's buffer resources covers."""
    import torch
    from kv_cache_token_amd.cache import EvictingCache
    budget, n_sink, recent = MAX_BUDGET, 4, 0
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    say("decode at budget %d, %s rows of %d" % (budget, dtype, Dd))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    k = torch.randn((1, budget, Dd), generator=gen, device="cuda").to(td)
    v = torch.randn((1, budget, Dd), generator=gen, device="cuda").to(td)
    k[0, 10] = 8.0           # the highest norm just after the sinks: evicted first under keep-low
    c = EvictingCache(1, 1, 1, budget, n_sink, recent, "low", "l2", dtype=dtype, head_dim=Dd)
    lock = oracle.OracleCache(1, Dd, dtype, budget, n_sink, recent, "low", "l2")
    c.update(k, v)
    lock.update(host_rows(k, [0], dtype), host_rows(v, [0], dtype), scores_in=host_rows(c.last_scores(), [0], "f32"))
    del k, v
    for t in range(3):
        kt = torch.randn((1, 1, Dd), generator=gen, device="cuda").to(td)
        vt = torch.randn((1, 1, Dd), generator=gen, device="cuda").to(td)
        c.update(kt, vt)
        lock.update(host_rows(kt, [0], dtype), host_rows(vt, [0], dtype),
                    scores_in=host_rows(c.last_scores(), [0], "f32"))
        torch.cuda.synchronize()
        assert_states_equal(gpu_state_arrays(c, [0]), lock, [0], "decode token %d at budget 2^21" % t)
    assert c.n_kept == budget and c.offset == budget + 3
