"""bench.py's host-side parts on the CPU: the one-GPU guard and the oracle
baseline leg (the GPU legs run on the device only)."""
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


@pytest.mark.parametrize("cid", [4, 3])
def test_oracle_baseline_leg_reports_its_sample(cid):
    import bench
    from kv_cache_token_amd import synth
    cfg = synth.CONFIGS[cid]
    tokens = len(cfg.scorers) * cfg.B * (256 if cid == 3 else cfg.tokens)
    wl = types.SimpleNamespace(cfg=cfg, tokens_per_step=tokens)
    cb = bench.cpu_baseline(wl, bench.recipe_bytes(cfg, 2), min_seconds=0.2)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0
    assert cb["value_1_thread"] > 0 and cb["cores"] >= 1
    assert "2 of %d groups" % cfg.G in cb["sample"]


def test_measured_traffic_matches_the_committed_counter_summaries():
    """bench.py's per-launch HBM traffic figures are the ones the committed
    rocprofv3 counter summaries derive, for the same kernel source hash."""
    import glob
    import re
    import bench
    names = {"c4": "c4_chunked_prefill_32k", "c3": "c3_decode_stream", "c5": "c5_keysvd_fallback_128k",
             "c2": "c2_qfilters_calibrated"}
    assert set(bench.MEASURED_TRAFFIC) == set(names)
    assert len(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.md"))) == len(names)
    for w, stem in names.items():
        text = open(os.path.join(ROOT, "profiles", stem + "_hbm_counters.md")).read()
        sha = re.search(r"Kernel source sha256\[:16\]: `([0-9a-f]{16})`", text).group(1)
        dom = int(re.search(r"Dominant kernel \(.*\): (\d+) calibrated HBM bytes per launch", text).group(1))
        mt = bench.MEASURED_TRAFFIC[w]
        assert mt["kernel_src_sha256_16"] == sha, w
        assert abs(mt["bytes_per_launch"] - dom) <= 1, w
        trace = open(os.path.join(ROOT, "profiles", stem + "_kernel_stats.md")).read()
        assert "`%s`" % sha in trace, w


def test_prefill_variants_resize_the_recipe_and_reach_the_oracle_leg():
    import dataclasses
    import bench
    from kv_cache_token_amd import synth
    ns = dict(workload="c4", dtype="f16", head_dim=64, budget=20000, chunk=16384, tokens=65536)
    cfg, text = bench.variant_config(types.SimpleNamespace(**ns))
    assert (cfg.dtype, cfg.D, cfg.budget, cfg.chunks) == ("f16", 64, 20000, (16384,) * 4)
    assert cfg.scorers == synth.CONFIGS[4].scorers and "f16" in text and "20000" in text
    same, text0 = bench.variant_config(types.SimpleNamespace(workload="c4", dtype=None, head_dim=None, budget=None,
                                                             chunk=None, tokens=None, layers=None))
    assert same is synth.CONFIGS[4] and text0 == ""
    one, text1 = bench.variant_config(types.SimpleNamespace(workload="c2", dtype=None, head_dim=None, budget=None,
                                                            chunk=256, tokens=None, layers=1))
    assert (one.L, one.H, one.G, one.chunks) == (1, 8, 8, (256,) * 16) and "1 layer," in text1
    for bad in (dict(ns, workload="c3"), dict(ns, tokens=1000), dict(ns, workload="c5", head_dim=256),
                dict(ns, layers=0)):
        with pytest.raises(SystemExit):
            bench.variant_config(types.SimpleNamespace(**bad))
    # the oracle leg runs the variant's own bytes (fp16 rows of 64 elements)
    small = dataclasses.replace(cfg, chunks=(300,) * 3, budget=500)
    wl = types.SimpleNamespace(cfg=small, tokens_per_step=2 * 900)
    cb = bench.cpu_baseline(wl, bench.recipe_bytes(small, 2), min_seconds=0.1)
    assert cb["value"] > 0


def _fake_workload(cfg, sample, filters):
    """What the oracle leg reads of a workload, without a GPU: one cache per
    scorer run over all layers (CPU tensors stand in for the filters)."""
    import torch
    from kv_cache_token_amd import api
    caches = []
    for sc in cfg.scorers:
        f = None if sc.mode == "l2" else torch.from_numpy(filters)
        caches.append(types.SimpleNamespace(mode=sc.mode, filters=f, L=cfg.L, B=cfg.B, H=cfg.H, D=cfg.D,
                                            score_shape=api.make_shape(cfg.L, cfg.B, cfg.H, cfg.dtype, cfg.D)))
    wl = types.SimpleNamespace(cfg=cfg, ranges=[(0, cfg.L)] * len(cfg.scorers), scorer_of=list(cfg.scorers),
                               sample=sample, bh=cfg.B * cfg.H, prefill_host=None, prefill_scores=[],
                               caches=caches, last_set=0, tokens_per_step=len(cfg.scorers) * cfg.tokens)
    wl.local = lambda l0, l1: [g - l0 * wl.bh for g in sample if l0 * wl.bh <= g < l1 * wl.bh]
    return wl


def test_oracle_leg_certifies_a_matching_state_and_flags_one_flipped_bit():
    """The bench's parity verdict: the oracle's rules replayed on captured
    scores give the captured final state -> bit_exact; one flipped bit in a
    kept K row, a stored score off by one ulp or a score outside the tolerance
    -> not certified.  (The captured data here comes from the oracle itself;
    on the GPU it is the device's.)"""
    import dataclasses
    import numpy as np
    import bench
    import oracle
    from kv_cache_token_amd import synth
    cfg = dataclasses.replace(synth.CONFIGS[4], L=1, H=4, chunks=(300, 300, 300), budget=400)
    sample = [0, 2, 3]
    f_lh = synth.filters_mu(cfg)
    wl = _fake_workload(cfg, sample, f_lh)
    inputs = bench.recipe_bytes(cfg, cfg.G)
    sel = [inputs["groups"].index(g) for g in sample]
    per_cache, states = [], []
    for sc in cfg.scorers:
        f = None if sc.mode == "l2" else np.stack([f_lh[0, g] for g in sample])
        keep = sc.keep if sc.mode == "l2" else "high"
        oc = oracle.OracleCache(len(sample), cfg.D, cfg.dtype, cfg.budget, cfg.n_sink, cfg.recent, keep, sc.mode,
                                f, sc.sign)
        calls = []
        for K, V in inputs["chunks"]:
            K, V = K[sel], V[sel]
            s = np.stack([oracle.score(K[i], sc.mode, None if f is None else f[i], sc.sign) for i in range(len(sel))])
            oc.update(K, V, scores_in=s)
            calls.append((K, V, s))
        per_cache.append(calls)
        n = int(oc.n[0])
        states.append((oc.k[:, :n].copy(), oc.v[:, :n].copy(), oc.s[:, :n].copy(), oc.pos[:, :n].copy()))
    captured = {0: (per_cache, states)}
    parity, cb = bench.oracle_leg(wl, captured, states, [0, 3], min_seconds=0.05)
    assert parity["bit_exact"] and parity["scores_within_tol"] and parity["states_compared"] == 4
    assert parity["groups"] == 3 and cb["value"] > 0 and "2 of 4 groups" in cb["sample"]
    bad = [tuple(x.copy() for x in st) for st in states]
    bad[1][0][2, 5, 7] ^= 1
    assert not bench.oracle_leg(wl, captured, bad, [0], min_seconds=0)[0]["bit_exact"]
    bad = [tuple(x.copy() for x in st) for st in states]
    bad[0][2].view(np.uint32)[1, 3] += 1
    assert not bench.oracle_leg(wl, captured, bad, [0], min_seconds=0)[0]["bit_exact"]
    K, V, s = per_cache[0][1]
    off = s.copy()
    off[0, 0] *= 1 + 1e-4
    moved = {0: ([[per_cache[0][0], (K, V, off), per_cache[0][2]], per_cache[1]], states)}
    assert not bench.oracle_leg(wl, moved, None, [0], min_seconds=0)[0]["scores_within_tol"]
