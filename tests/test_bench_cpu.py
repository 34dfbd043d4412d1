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
    cb = bench.cpu_baseline(wl, 2, min_seconds=0.2)
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
                                                             chunk=None, tokens=None))
    assert same is synth.CONFIGS[4] and text0 == ""
    for bad in (dict(ns, workload="c3"), dict(ns, tokens=1000), dict(ns, workload="c5", head_dim=256)):
        with pytest.raises(SystemExit):
            bench.variant_config(types.SimpleNamespace(**bad))
    # the oracle leg runs the variant's own bytes (fp16 rows of 64 elements)
    small = dataclasses.replace(cfg, chunks=(300,) * 3, budget=500)
    wl = types.SimpleNamespace(cfg=small, tokens_per_step=2 * 900)
    cb = bench.cpu_baseline(wl, 2, min_seconds=0.1)
    assert cb["value"] > 0
