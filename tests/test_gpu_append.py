"""kv_score_append (a call that evicts nothing: score and append in one pass)
against the two calls it replaces, qf_score_keys then the in-place
kv_compact_gather, through the C ABI: the cache buffers (every row, the rows
past the appended ones included) and the scores are bit-identical for every
element type, head dim, scorer and sign, for an empty and a partly filled
cache, ragged row counts and per-group filters; and the scores match the
oracle's within the tolerance."""
import numpy as np
import pytest

import oracle
from kv_cache_token_amd import synth
from tests.gpu_util import assert_scores_close, oracle_scores, score_scales

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


CASES = [(dt, Dd, mode, sign, n_kept, S)
         for dt, Dd in (("bf16", 128), ("f16", 64), ("f32", 256), ("bf16", 256), ("f32", 64))
         for mode, sign in (("l2", 1), ("proj", 1), ("proj", -1))
         for n_kept, S in ((0, 1000), (37, 333), (100, 2))]


@pytest.mark.parametrize("dt,Dd,mode,sign,n_kept,S", CASES, ids=[str(c) for c in CASES])
def test_score_append_equals_score_then_append(dt, Dd, mode, sign, n_kept, S):
    import torch
    from kv_cache_token_amd import api
    L, B, H, budget = 2, 2, 3, 1500
    G = L * B * H
    rng = np.random.default_rng(n_kept + S + Dd)
    f = torch.from_numpy(rng.standard_normal((L, H, Dd)).astype(np.float32)).cuda() if mode == "proj" else None
    K = synth.custom_keys((G, S, Dd), 500 + S, dt)
    V = synth.custom_keys((G, S, Dd), 600 + S, dt)
    kt, vt = synth.host_to_torch(K, dt).cuda(), synth.host_to_torch(V, dt).cuda()
    td = api.torch_dtype(api.dtype_code(dt))
    base = [synth.host_to_torch(synth.custom_keys((G, budget, Dd), 700, dt), dt).cuda(),
            synth.host_to_torch(synth.custom_keys((G, budget, Dd), 701, dt), dt).cuda(),
            torch.from_numpy(rng.standard_normal((G, budget)).astype(np.float32)).cuda(),
            torch.from_numpy(rng.integers(0, 10 ** 6, (G, budget)).astype(np.int32)).cuda()]
    assert base[0].dtype == td
    shape, params = api.make_shape(L, B, H, dt, Dd), api.make_params(budget, 4, 0, "high" if mode == "proj" else "low")
    pos_base = 12345
    ref = [x.clone() for x in base]
    s_ref = torch.full((G, S), float("nan"), device="cuda")
    api.qf_score_keys(kt, shape, S, mode, f, sign, s_ref)
    api.kv_compact_gather(*ref, kt, vt, s_ref, pos_base, None, shape, n_kept, S, params, *ref)
    got = [x.clone() for x in base]
    s_got = torch.full((G, S), float("nan"), device="cuda")
    api.kv_score_append(kt, vt, shape, S, mode, f, sign, pos_base, n_kept, params, *got, s_got)
    no_copy = [x.clone() for x in base]
    api.kv_score_append(kt, vt, shape, S, mode, f, sign, pos_base, n_kept, params, *no_copy, None)
    torch.cuda.synchronize()
    for a, b, c in zip(ref, got, no_copy):
        assert torch.equal(_bits(a), _bits(b)) and torch.equal(_bits(a), _bits(c))
    assert torch.equal(s_ref.view(torch.int32), s_got.view(torch.int32))
    fg = None if f is None else np.stack([f.cpu().numpy()[g // (B * H), g % H] for g in range(G)])
    s_o = oracle_scores(K, dt, mode, fg, sign)
    assert_scores_close(s_got.cpu().numpy(), s_o, score_scales(K, dt, mode, s_o, fg), "append")


def test_score_append_with_per_group_filters_and_a_stream():
    """The fallback's layout: one filter per (layer, batch, head) group,
    described as L' = L*B, B' = 1; on a side stream."""
    import torch
    from kv_cache_token_amd import api
    L, B, H, D, S, budget = 2, 3, 4, 128, 500, 600
    G = L * B * H
    f = torch.from_numpy(np.random.default_rng(9).standard_normal((L * B, H, D)).astype(np.float32)).cuda()
    K = synth.custom_keys((G, S, D), 91, "bf16")
    kt = synth.host_to_torch(K, "bf16").cuda()
    shape = api.make_shape(L * B, 1, H, "bf16")
    params = api.make_params(budget, 4, 0, "high")
    st = torch.cuda.Stream()
    bufs = [torch.zeros((G, budget, D), dtype=torch.bfloat16, device="cuda"),
            torch.zeros((G, budget, D), dtype=torch.bfloat16, device="cuda"),
            torch.zeros((G, budget), device="cuda"), torch.zeros((G, budget), dtype=torch.int32, device="cuda")]
    torch.cuda.synchronize()
    api.kv_score_append(kt, kt.flip(1).contiguous(), shape, S, "proj", f, -1, 0, 0, params, *bufs, None, stream=st)
    st.synchronize()
    s = bufs[2][:, :S].cpu().numpy()
    fg = f.reshape(G, D).cpu().numpy()
    want = np.stack([oracle.score(K[g], "proj", fg[g], -1) for g in range(G)])
    assert_scores_close(s, want, score_scales(K, "bf16", "proj", want, fg), "per-group filters")
    assert np.array_equal(bufs[3][:, :S].cpu().numpy(), np.tile(np.arange(S, dtype=np.int32), (G, 1)))
    assert np.array_equal(synth.torch_to_host(bufs[0][:, :S], "bf16"), K)
