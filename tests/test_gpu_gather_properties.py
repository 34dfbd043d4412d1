"""Property-based parity of the compaction (kv_compact_gather) with a numpy
gather on drawn cases: any strictly increasing list of budget rows out of the
concatenation (not only the ones a selection would pick), every element type
and head dim, kept and incoming row counts from zero upward, ragged group
counts, and the in-place append of a call that evicts nothing.  K and V bytes,
scores and positions must equal out[j] = concat[keep_idx[j]] bit for bit, and
rows past the output must stay untouched.  Hypothesis runs derandomised."""
import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

from kv_cache_token_amd import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from kv_cache_token_amd import _lib
    _lib.lib()


@st.composite
def case(draw):
    dtype = draw(st.sampled_from(["bf16", "f16", "f32"]))
    Dd = draw(st.sampled_from([64, 128, 256]))
    G = draw(st.integers(1, 5))
    budget = draw(st.integers(1, 3000))
    n_kept = draw(st.integers(0, budget))
    S = draw(st.integers(0, 3000))
    in_place = draw(st.booleans()) and n_kept + S <= budget
    seed = draw(st.integers(0, 2 ** 31 - 1))
    return dtype, Dd, G, budget, n_kept, S, in_place, seed


def _bits(t):
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    return t.view(torch.int32) if t.dtype == torch.float32 else t


@settings(max_examples=100, deadline=None, derandomize=True)
@given(case())
def test_compaction_is_the_indexed_gather(c):
    import torch
    from kv_cache_token_amd import api
    dtype, Dd, G, budget, n_kept, S, in_place, seed = c
    rng = np.random.default_rng(seed)
    n_total = n_kept + S
    n_out = min(n_total, budget)
    evict = n_total > budget
    say("gather case %s" % (c,))
    td = api.torch_dtype(api.dtype_code(dtype))
    kept = [synth.host_to_torch(synth.custom_keys((G, budget, Dd), seed % 1000, dtype), dtype).cuda(),
            synth.host_to_torch(synth.custom_keys((G, budget, Dd), seed % 1000 + 1, dtype), dtype).cuda(),
            torch.from_numpy(rng.standard_normal((G, budget)).astype(np.float32)).cuda(),
            torch.from_numpy(rng.integers(0, 1 << 30, (G, budget)).astype(np.int32)).cuda()]
    kn = synth.host_to_torch(synth.custom_keys((G, max(S, 1), Dd), seed % 1000 + 2, dtype), dtype).cuda()
    vn = synth.host_to_torch(synth.custom_keys((G, max(S, 1), Dd), seed % 1000 + 3, dtype), dtype).cuda()
    sn = torch.from_numpy(rng.standard_normal((G, max(S, 1))).astype(np.float32)).cuda()
    idx = np.zeros((G, budget), dtype=np.int32)
    for g in range(G):
        rows = np.sort(rng.choice(n_total, size=n_out, replace=False)) if evict else np.arange(n_total)
        idx[g, :n_out] = rows
    keep_idx = torch.from_numpy(idx).cuda()
    params = api.make_params(budget, 0, 0, "high")
    shape = api.make_shape(1, 1, G, dtype, Dd)
    pos_base = int(rng.integers(0, 1 << 30))
    before = [x.clone() for x in kept]
    if in_place:
        out = kept
    else:
        out = [torch.full_like(x, 0) for x in kept]
        for x in out:
            x.view(torch.uint8).fill_(0xA5)
    snapshot = [x.clone() for x in out]
    api.kv_compact_gather(*kept, kn if S else None, vn if S else None, sn if S else None, pos_base,
                          keep_idx if evict else None, shape, n_kept, S, params, *out)
    torch.cuda.synchronize()
    cat_k = torch.cat([before[0][:, :n_kept], kn[:, :S]], dim=1)
    cat_v = torch.cat([before[1][:, :n_kept], vn[:, :S]], dim=1)
    cat_s = torch.cat([before[2][:, :n_kept], sn[:, :S]], dim=1)
    cat_p = torch.cat([before[3][:, :n_kept],
                       (pos_base + torch.arange(S, dtype=torch.int32, device="cuda")).repeat(G, 1)], dim=1)
    ix = keep_idx[:, :n_out].long()
    for name, cat, got, snap in zip(("k", "v", "s", "pos"), (cat_k, cat_v, cat_s, cat_p), out, snapshot):
        if cat.dim() == 3:
            want = torch.gather(cat, 1, ix[:, :, None].expand(-1, -1, Dd))
        else:
            want = torch.gather(cat, 1, ix)
        assert torch.equal(_bits(got[:, :n_out]), _bits(want)), name
        assert torch.equal(_bits(got[:, n_out:]), _bits(snap[:, n_out:])), name + " past the output"
