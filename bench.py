#!/usr/bin/env python3
"""Benchmark of the query-free KV-cache eviction step on one MI355X.

Workload (one step): the chunked long prefill of 28 layers x 8 KV heads
(224 groups), head_dim 128, bf16 K/V, 32768 tokens absorbed in 4096-token
chunks into a cache of budget 4096 with 4 sinks, once with the L2-norm scorer
(keep lowest) and once with the Q-Filters projection scorer on the planted
direction with sign -1.  Each chunk is one score + select + compact pass over
all 224 groups.  Inputs are seeded synthetic tensors resident in HBM before the
timed region; the step starts from an empty cache each time.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value       tokens absorbed per second, summed over the two scorer runs
  roofline    the compaction (gather) kernel of the evicting calls: algorithmic
              bytes per launch / its mean duration from HIP events recorded on the
              launch stream inside the timed region, against 8 TB/s
  cpu_baseline the oracle (plain C, OpenMP) on a sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
D = 128
KERNEL_SRC = os.path.join(ROOT, "kv_cache_token_amd", "csrc", "kvx_device.hip")
# HBM bytes per evicting compaction launch, from the two rocprofv3 counter runs
# (FETCH_SIZE x 2.0 and WRITE_SIZE x 1.0, factors from a 1 GiB device copy) in
# profiles/c4_chunked_prefill_32k_hbm_counters.md, valid only for the kernel
# source they were taken on.
MEASURED_TRAFFIC = {"kernel_src_sha256_16": "fcba0c27a0cb1391", "bytes_per_launch": 977377568}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_workload(torch, stream):
    from kv_cache_token_amd import synth
    from kv_cache_token_amd.cache import EvictingCache
    cfg = synth.CONFIGS[4]
    with torch.cuda.stream(stream):
        mus = synth.device_mus(cfg)
        blocks = [synth.fill_device(cfg, S, 1000 + c, mus=mus) for c, S in enumerate(cfg.chunks)]
        f = torch.from_numpy(synth.filters_mu(cfg)).cuda()
        caches = []
        for sc in cfg.scorers:
            keep = sc.keep if sc.mode == "l2" else "high"
            caches.append(EvictingCache(cfg.L, cfg.B, cfg.H, cfg.budget, cfg.n_sink, cfg.recent, keep, sc.mode,
                                        f if sc.mode == "proj" else None, sc.sign, cfg.dtype, stream=stream))
        plans = [c.plan(blocks) for c in caches]
    torch.cuda.synchronize()
    return cfg, blocks, caches, plans


def algorithmic_bytes(torch, cfg, caches, plans, stream):
    """Run each plan once call by call, reading keep_idx after every selection,
    and count the bytes the method must move (per the workload's own survivors):
    per group and call, S*Row (read incoming K) + 4*n_kept (stored scores)
    + m_k*2*(2*Row+8) (kept survivors whose row changes: read and write K, V,
    score, position) + m_n*(3*Row+8) (incoming survivors: read V, write K, V,
    score, position).  Also the gather kernel's own bytes per evicting launch:
    every output row reads K, V, score and its index and writes K, V, score and
    position: 4*Row+16 bytes."""
    row = D * 2
    step_bytes = 0
    gather_bytes = []
    for cache, plan in zip(caches, plans):
        state = {"n_kept": 0}
        S_of = list(cfg.chunks)
        call_chunk = []
        c = -1
        for name in plan.names:
            if name == "qf_score_keys":
                c += 1
            call_chunk.append(c)

        def hook(i, name, when, cache=cache, state=state):
            nonlocal step_bytes
            if when != "after":
                return
            ch = call_chunk[i]
            S = S_of[ch]
            nk = state["n_kept"]
            if name == "kv_compact_gather":
                G = cache.G
                if nk + S <= cache.budget:        # append in place
                    m_k, m_n = 0, S
                    step_bytes += G * (S * row + 4 * nk + m_n * (3 * row + 8))
                else:
                    torch.cuda.synchronize()
                    idx = cache.keep_idx.to(torch.int64)
                    j = torch.arange(idx.shape[1], device=idx.device)[None, :]
                    m_k = int(((idx < nk) & (idx != j)).sum())
                    m_n = int((idx >= nk).sum())
                    step_bytes += G * (S * row + 4 * nk) + m_k * 2 * (2 * row + 8) + m_n * (3 * row + 8)
                    gather_bytes.append(G * cache.budget * (4 * row + 16))
                state["n_kept"] = min(nk + S, cache.budget)

        with torch.cuda.stream(stream):
            plan.run(hook)
        torch.cuda.synchronize()
    return step_bytes, gather_bytes


def cpu_baseline(cfg, n_groups):
    """The oracle as it stands, on a sample of the same workload (exact seeded
    host bytes of n_groups groups, both scorer runs over the whole stream)."""
    import numpy as np

    import oracle
    from kv_cache_token_amd import synth
    sample = synth.sample_groups(cfg, n_groups)
    t0 = time.perf_counter()
    chunks = [synth.batch_chunk(cfg, sample, c) for c in range(len(cfg.chunks))]
    log("cpu baseline: generated %d groups in %.1f s" % (len(sample), time.perf_counter() - t0))
    f_lh = synth.filters_mu(cfg)
    fs = np.stack([f_lh[cfg.group_lbh(g)[0], cfg.group_lbh(g)[2]] for g in sample])
    caches = []
    for sc in cfg.scorers:
        keep = sc.keep if sc.mode == "l2" else "high"
        caches.append(oracle.OracleCache(len(sample), D, cfg.dtype, cfg.budget, cfg.n_sink, cfg.recent, keep,
                                         sc.mode, fs if sc.mode == "proj" else None, sc.sign))
    t0 = time.perf_counter()
    for oc in caches:
        for K, V in chunks:
            oc.update(K, V)
    t = time.perf_counter() - t0
    tokens = len(cfg.scorers) * cfg.tokens * len(sample) / cfg.G     # workload-equivalent tokens
    return {"value": tokens / t, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d groups, both scorer runs over the full %d-token stream (%.2f s)"
                      % (len(sample), cfg.G, cfg.tokens, t)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-groups", type=int, default=32, help="groups in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay each step as one captured HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run the same "
            "step on its own groups); run with --gpus 1")
        sys.exit(2)

    import torch
    from kv_cache_token_amd import _lib
    _lib.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_name = torch.cuda.get_device_name(0)
    stream = torch.cuda.Stream()
    cfg, blocks, caches, plans = build_workload(torch, stream)
    log("workload ready on %s: %d groups, %d chunks of %d" % (dev_name, cfg.G, len(cfg.chunks), cfg.chunks[0]))

    if args.copy_calibration:
        with torch.cuda.stream(stream):
            src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step_bytes, gather_bytes = algorithmic_bytes(torch, cfg, caches, plans, stream)
    log("algorithmic bytes per step: %.3f GB; gather launches per step: %d" % (step_bytes / 1e9, len(gather_bytes)))

    def step(hook=None):
        for p in plans:
            p.run(hook)

    graph = None
    if args.graph:
        with torch.cuda.stream(stream):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay() if graph else step()
    torch.cuda.synchronize()

    # Timed region: K steps; the compaction launches of evicting calls are
    # bracketed by events on the launch stream.
    gather_events = []
    ev = torch.cuda.Event

    def hook(i, name, when):
        if name != "kv_compact_gather":
            return
        e = ev(enable_timing=True)
        e.record(stream)
        gather_events.append((i, when, e))

    start, end = ev(enable_timing=True), ev(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            if graph:
                graph.replay()
            else:
                step(hook)
    end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps

    # per-launch gather durations (evicting calls only: every call after the first chunk)
    gather_ms = []
    if gather_events:
        for k in range(0, len(gather_events), 2):
            (i0, w0, e0), (i1, w1, e1) = gather_events[k], gather_events[k + 1]
            assert w0 == "before" and w1 == "after" and i0 == i1
            gather_ms.append((i0, e0.elapsed_time(e1)))
    evict_ms = [ms for n, (i, ms) in enumerate(gather_ms) if (n % len(cfg.chunks)) != 0]
    roof = None
    if evict_ms:
        mean_ms = sum(evict_ms) / len(evict_ms)
        bytes_per_launch = sum(gather_bytes) / len(gather_bytes)
        achieved = bytes_per_launch / (mean_ms * 1e-3) / 1e9
        import hashlib
        sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]
        traffic = MEASURED_TRAFFIC["bytes_per_launch"] if sha == MEASURED_TRAFFIC["kernel_src_sha256_16"] else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic, "traffic_unit": "bytes/launch",
                "kernel": "kv_compact_gather (evicting calls)", "launches": len(evict_ms),
                "mean_launch_us": round(mean_ms * 1e3, 2), "algorithmic_bytes_per_launch": int(bytes_per_launch)}
    tokens_per_step = len(cfg.scorers) * cfg.tokens
    value = tokens_per_step / (ms_per_step * 1e-3)
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "evicted-cache tokens/sec (score+select+compact), achieved HBM GB/s vs peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded anisotropic keys drift*mu + N(0,0.25), V ~ N(0,1); HBM-resident)",
        "config": {"workload": "c4_chunked_prefill_32k: 28 layers x 8 KV heads x head_dim 128 (224 groups), bf16, "
                               "32768 tokens in 4096-token chunks, budget 4096, 4 sinks, recent 0; "
                               "L2-norm keep-low run + Q-Filters (planted filter, sign -1) run",
                   "groups": cfg.G, "tokens_per_run": cfg.tokens, "chunk": cfg.chunks[0], "budget": cfg.budget,
                   "runs_per_step": len(cfg.scorers), "graph": bool(graph), "device": dev_name},
        "step_algorithmic_GBps": round(step_gbps, 1), "step_frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
        "step_algorithmic_bytes": int(step_bytes),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_groups)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
