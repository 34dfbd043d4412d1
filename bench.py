#!/usr/bin/env python3
"""Benchmark of the query-free KV-cache eviction step on one MI355X.

Default workload (one step): the chunked long prefill of 28 layers x 8 KV heads
(224 groups), head_dim 128, bf16 K/V, 32768 tokens absorbed in 4096-token chunks
into a cache of budget 4096 with 4 sinks, once with the L2-norm scorer (keep
lowest) and once with the Q-Filters projection scorer on the planted direction
with sign -1.  Each chunk is one score + select + compact pass over all groups.
Inputs are seeded synthetic tensors resident in HBM before the timed region; the
step starts from an empty cache each time.

Other workloads (--workload): c2 (one 4096-token block, budget 512,
projection), c3 (7168 groups, a full cache of budget 2048, then 256
single-token decode steps with a recent window of 512; the cache is restored
from a device snapshot, untimed, before each step), c5 (256 groups, 131072
tokens in 8192-token chunks, budget 8192, key-SVD fallback filters estimated
before the timed region; the estimate's own time is reported beside), qcal (the
query-SVD calibration of a 28-layer model with 24 query heads over 8 KV heads,
3000 samples per query head, on the device; a once-per-model step outside the
eviction path, reported with its own metric).  --dtype, --head-dim, --budget,
--chunk and --tokens run a prefill workload's recipe at other sizes (fp16 or
fp32 K/V, head dims 64 and 256, budgets past the on-chip selection); the
variant is named in config.workload.

Prints ONE JSON line on stdout (everything else goes to stderr):
  value        tokens absorbed per second over the whole step (all runs), from
               the median of the timed steps (each step bracketed by its own
               HIP events on the launch stream; mean, min and max beside it)
  roofline     the dominant kernel (the compaction of evicting calls for
               prefill, the in-place decode kernel for c3): its share of the
               step's algorithmic bytes (what the method must move: survivors
               whose row changes read and written, incoming survivors' V read
               and K, V, score, position written; decode adds the stored
               scores it ranks) per launch over its mean duration from HIP
               events recorded on the launch stream around every call, in a
               second timed pass; the bytes the kernel itself moves and the
               rocprofv3 counters' HBM traffic beside them.  (A call that
               evicts nothing scores and appends in one pass, kv_score_append,
               and has no compaction launch.)
  parity       the oracle's verdict on the sampled groups: an untimed pass
               copies back their input bytes and the GPU's scores of every
               call; the oracle replays its selection and compaction on those
               scores, and its final kept rows, K/V bytes, stored scores and
               positions must equal the GPU's bit for bit, both after that
               pass and after the timed steps; its own fp64-derived scores
               must lie within 1e-5 of the GPU's (of the norm, or of
               sum_d |k_d f_d|).  A mismatch exits with status 1.
  cpu_baseline the oracle (plain C, OpenMP) on the same input bytes of a
               sample of groups, repeated to about 10 s, with its
               single-thread rate beside
  beside them  head_tokens_per_s, the step's algorithmic GB/s, the kernels'
               mean launch times, the library's own device-copy rate and (c2,
               c4) the same step launched layer by layer; --no-extras skips the
               last two.  --streams / --split run independent caches
               concurrently (--streams 2 puts the two scorer runs of c4 side
               by side).  The default line uses one stream, so that the timed
               steps, the per-kernel pass behind the roofline and a kernel
               trace of the same command all see each kernel running alone.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
D = 128
KERNEL_SRC = os.path.join(ROOT, "kv_cache_token_amd", "csrc", "kvx_device.hip")
# Calibrated HBM bytes per launch of the dominant kernel, from the two rocprofv3
# counter runs (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0; factors from a 1 GiB device
# copy) summarised in profiles/, valid only for the kernel source they were
# taken on (sha256 prefix of kvx_device.hip).
MEASURED_TRAFFIC = {
    "c4": {"kernel_src_sha256_16": "79c3f6f631ddb13a", "bytes_per_launch": 964555599},
    "c3": {"kernel_src_sha256_16": "79c3f6f631ddb13a", "bytes_per_launch": 9128278411},
    "c5": {"kernel_src_sha256_16": "79c3f6f631ddb13a", "bytes_per_launch": 2204763726},
    "c2": {"kernel_src_sha256_16": "79c3f6f631ddb13a", "bytes_per_launch": 122618569},
}
DESCRIPTIONS = {
    "c2": "c2_qfilters_calibrated: 28 layers x 8 KV heads x 128 (224 groups), bf16, one 4096-token block, "
          "budget 512, 4 sinks; projection on the planted filter, sign +1",
    "c3": "c3_decode_stream: 32 sequences x 28 layers x 8 KV heads x 128 (7168 groups), bf16, cache full at "
          "budget 2048, then 256 single-token steps; L2 keep-low, 4 sinks, recent 512",
    "c4": "c4_chunked_prefill_32k: 28 layers x 8 KV heads x head_dim 128 (224 groups), bf16, 32768 tokens in "
          "4096-token chunks, budget 4096, 4 sinks, recent 0; L2-norm keep-low run + Q-Filters (planted filter, "
          "sign -1) run",
    "c5": "c5_keysvd_fallback_128k: 32 layers x 8 KV heads x 128 (256 groups), bf16, 131072 tokens in 8192-token "
          "chunks, budget 8192, 4 sinks; projection on key-SVD fallback filters (first 128 keys, estimated "
          "before timing), sign +1",
    "qcal": "query-SVD calibration: 28 layers x 24 query heads over 8 KV heads x 128, bf16 activations, 3000 "
            "samples per query head; fp64 Gram + power iteration + GQA averaging per (layer, KV head)",
}
PEAK_FP64_TFLOPS = 78.6


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Workload:
    """One plan per scorer run over HBM-resident seeded inputs; with split > 1
    each run's groups are divided by layer into that many independent caches
    (the step is per group), spread over the streams.  `sample` lists the
    groups whose bytes and scores the parity pass copies back."""

    def __init__(self, torch, name, streams, split=1, cfg=None, sample=()):
        from kv_cache_token_amd import synth
        from kv_cache_token_amd.cache import EvictingCache
        cid = int(name[1:])
        self.name, self.cfg, self.streams = name, cfg or synth.CONFIGS[cid], streams
        cfg = self.cfg
        self.row = cfg.D * (4 if cfg.dtype == "f32" else 2)   # bytes of one K or V row
        self.sample = sorted(sample)
        with torch.cuda.stream(streams[0]):
            mus = synth.device_mus(cfg) if cfg.keys == "aniso" else None
            if cid == 3:
                prefill = synth.fill_device(cfg, cfg.chunks[0], 3000)
                kd, vd = synth.fill_device(cfg, 256, 3001)
                kd, vd = kd.transpose(0, 1).contiguous(), vd.transpose(0, 1).contiguous()
                self.blocks = [(kd[t].unsqueeze(1), vd[t].unsqueeze(1)) for t in range(256)]
            else:
                self.blocks = [synth.fill_device(cfg, S, 1000 * cid + c, mus=mus) for c, S in enumerate(cfg.chunks)]
            f_mu = torch.from_numpy(synth.filters_mu(cfg)).cuda() if cfg.keys == "aniso" else None
        self.f_mu = f_mu
        if split < 1 or cfg.L % split:
            raise ValueError("split must divide the layer count %d" % cfg.L)
        per = cfg.L // split
        self.bh = bh = cfg.B * cfg.H

        def part(blocks, l0, l1):
            return [(k[l0 * bh:l1 * bh], v[l0 * bh:l1 * bh]) for k, v in blocks]

        self.caches, self.plans, self.snapshots, self.ranges, self.scorer_of = [], [], [], [], []
        self.prefill_host, self.prefill_scores = None, []
        if cid == 3:
            self.prefill_host = (host_rows(prefill[0], self.sample, cfg.dtype),
                                 host_rows(prefill[1], self.sample, cfg.dtype))
        for i, sc in enumerate(cfg.scorers):
            keep = sc.keep if sc.mode == "l2" else "high"
            for p in range(split):
                l0, l1 = p * per, (p + 1) * per
                st = streams[(i * split + p) % len(streams)]
                c = EvictingCache(per, cfg.B, cfg.H, cfg.budget, cfg.n_sink, cfg.recent, keep, sc.mode,
                                  f_mu[l0:l1] if sc.filt == "mu" else None, sc.sign, cfg.dtype, stream=st,
                                  calib_tokens=cfg.calib_tokens, calib_keys=cfg.calib_keys, head_dim=cfg.D)
                blocks = part(self.blocks, l0, l1)
                with torch.cuda.stream(st):
                    if sc.filt == "keysvd":       # freeze the fallback filters once, outside the timed step
                        c.update(*blocks[0])
                        c.reset(keep_filters=True)
                    if cid == 3:                  # the decode step starts from a full cache
                        c.update(*part([prefill], l0, l1)[0])
                        self.prefill_scores.append(host_rows(c.last_scores(), self.local(l0, l1)))
                        self.snapshots.append([x.clone() for x in c.buffers()])
                        self.plans.append(c.plan(blocks, keep_state=True))
                    else:
                        self.plans.append(c.plan(blocks))
                self.caches.append(c)
                self.ranges.append((l0, l1))
                self.scorer_of.append(sc)
        # Inputs that fit a few times in the 256 MB last-level cache (c2) are
        # rotated between two seeded sets, so that a step never re-reads the
        # previous step's inputs from that cache.
        self.plan_sets = [self.plans]
        self.block_sets = [self.blocks]
        in_bytes = sum(2 * k.numel() * k.element_size() for k, _ in self.blocks)
        if in_bytes < (1 << 30) and not self.snapshots and all(sc.filt != "keysvd" for sc in cfg.scorers):
            with torch.cuda.stream(streams[0]):
                alt = [synth.fill_device(cfg, S, 1000 * cid + 500 + c, mus=mus) for c, S in enumerate(cfg.chunks)]
            self.plan_sets.append([c.plan(part(alt, l0, l1)) for c, (l0, l1) in zip(self.caches, self.ranges)])
            self.block_sets.append(alt)
        self._turn = 0
        torch.cuda.synchronize()
        self.tokens_per_step = len(cfg.scorers) * cfg.B * sum(b[0].shape[1] for b in self.blocks)
        self.calls_per_step = sum(len(p.calls) for p in self.plans)
        self.dominant = "kv_evict_one_inplace" if cid == 3 else "kv_compact_gather"

    def local(self, l0, l1):
        """Indices, inside the cache of layers [l0, l1), of the sampled groups it holds."""
        return [g - l0 * self.bh for g in self.sample if l0 * self.bh <= g < l1 * self.bh]

    def restore(self):
        """Put back the cache contents the plans start from (untimed)."""
        for c, snap in zip(self.caches, self.snapshots):
            with self._torch.cuda.stream(c.stream):
                for d, s in zip(c.buffers(), snap):
                    d.copy_(s)

    @property
    def _torch(self):
        import torch
        return torch

    @property
    def last_set(self) -> int:
        """Index of the plan set the last step ran."""
        return (self._turn - 1) % len(self.plan_sets)

    def step(self, hook=None):
        plans = self.plan_sets[self._turn % len(self.plan_sets)]
        self._turn += 1
        for p in plans:
            p.run(hook)


def host_rows(t, groups, dtype=None):
    """Host copy of t[groups]: K/V rows of `dtype` as their stored bytes
    (uint16 for bf16 / f16), other tensors as they are (dtype None)."""
    import torch
    from kv_cache_token_amd import synth
    idx = torch.as_tensor(list(groups), dtype=torch.long, device=t.device)
    sel = t.index_select(0, idx)
    return synth.torch_to_host(sel, dtype) if dtype else sel.cpu().numpy()


def sampled_state(wl):
    """Host copies (k, v, s, pos) of the sampled groups' kept rows, per cache."""
    out = []
    for c, (l0, l1) in zip(wl.caches, wl.ranges):
        k, v, s, p = c.kept()
        loc = wl.local(l0, l1)
        out.append((host_rows(k, loc, c.dtype_name), host_rows(v, loc, c.dtype_name), host_rows(s, loc),
                    host_rows(p, loc)))
    return out


def capture_pass(torch, wl):
    """Untimed: run every plan set once, call by call, and copy back, for the
    sampled groups, the input bytes and the GPU's scores of every call and the
    final kept state.  Returns {set: [per cache: (calls, state)]}, calls being
    (K, V, scores) per block."""
    out = {}
    for si, plans in enumerate(wl.plan_sets):
        wl.restore()
        torch.cuda.synchronize()
        per_cache, rows = [], {}   # rows: one host copy of each block per layer range (the runs share them)
        for ci, (plan, c, (l0, l1)) in enumerate(zip(plans, wl.caches, wl.ranges)):
            bh = wl.bh
            blocks = [(k[l0 * bh:l1 * bh], v[l0 * bh:l1 * bh]) for k, v in wl.block_sets[si]]
            loc = wl.local(l0, l1)
            calls, st = [], {"blk": 0}

            def hook(i, name, when, c=c, loc=loc, blocks=blocks, calls=calls, st=st, l0=l0):
                if when != "after" or name not in ("qf_score_keys", "kv_score_append"):
                    return
                b = st["blk"]
                k, v = blocks[b]
                if (l0, b) not in rows:
                    rows[(l0, b)] = (host_rows(k, loc, c.dtype_name), host_rows(v, loc, c.dtype_name))
                calls.append(rows[(l0, b)] + (host_rows(c.last_scores()[:, :k.shape[1]], loc),))
                st["blk"] += 1

            with torch.cuda.stream(c.stream):
                plan.run(hook)
            torch.cuda.synchronize()
            per_cache.append(calls)
        out[si] = (per_cache, sampled_state(wl))
    wl._turn = len(wl.plan_sets)   # the next step starts with set 0 again
    return out


def algorithmic_bytes(torch, wl):
    """Run each plan once call by call and count the bytes the method must
    move, per group and call: S*Row (read incoming K) + 4*n_kept (stored
    scores) + m_k*2*(2*Row+8) (kept survivors whose row changes: read and write
    K, V, score, position) + m_n*(3*Row+8) (incoming survivors: read V, write
    K, V, score, position).  Returns the step's total and, per launch of the
    dominant kernel, (its share of those bytes, the bytes it moves itself):
    an evicting compaction's share is the two survivor terms (it moves
    4*Row+16 per output row: K, V, score and index read, K, V, score and
    position written); the decode kernel's share adds the 4*n_kept of the
    stored scores it ranks (it reads 4 B per candidate, moves each shifted row
    (2*(2*Row+8)) and reads and writes the incoming row (2*Row+4 + 2*Row+8))."""
    total, dom = 0, []
    ROW = wl.row
    wl.restore()
    for cache, plan in zip(wl.caches, wl.plans):
        st = {"n_kept": plan.start[0], "S": 0, "pos": None}
        G = cache.G

        def hook(i, name, when, cache=cache, st=st):
            nonlocal total
            if name in ("qf_score_keys", "kv_score_append") and when == "after":
                st["S"] = cache.last_scores().shape[1]
            if name == "qf_score_keys":
                return
            S, nk = st["S"], st["n_kept"]
            if name == "kv_score_append":
                if when == "after":   # nothing evicted: every incoming row appended
                    total += G * (S * ROW + 4 * nk + S * (3 * ROW + 8))
                    st["n_kept"] = nk + S
                return
            if name == "kv_evict_one_inplace":
                if when == "before":
                    torch.cuda.synchronize()
                    st["pos"] = cache.buffers()[3].clone()
                    return
                torch.cuda.synchronize()
                if nk < cache.budget:
                    total += G * (ROW + 4 * nk + (3 * ROW + 8))
                    dom.append((G * (4 * nk + 3 * ROW + 8), G * (4 * ROW + 12)))
                else:
                    diff = st["pos"] != cache.buffers()[3]
                    changed = diff.any(dim=1)
                    first = diff.to(torch.int32).argmax(dim=1).to(torch.int64)
                    victim = torch.where(changed, first, torch.full_like(first, cache.budget))
                    m_k = int((cache.budget - 1 - victim).clamp(min=0).sum())
                    m_n = int(changed.sum())
                    moved = m_k * 2 * (2 * ROW + 8)
                    total += G * (ROW + 4 * nk) + moved + m_n * (3 * ROW + 8)
                    cands = cache.budget + 1 - cache.recent - cache.n_sink
                    dom.append((G * 4 * nk + moved + m_n * (3 * ROW + 8),
                                G * 4 * cands + moved + m_n * (4 * ROW + 12)))
                st["n_kept"] = min(nk + 1, cache.budget)
            elif name == "kv_compact_gather" and when == "after":
                if nk + S <= cache.budget:
                    total += G * (S * ROW + 4 * nk + S * (3 * ROW + 8))
                else:
                    torch.cuda.synchronize()
                    idx = cache.keep_idx.to(torch.int64)
                    j = torch.arange(idx.shape[1], device=idx.device)[None, :]
                    m_k = int(((idx < nk) & (idx != j)).sum())
                    m_n = int((idx >= nk).sum())
                    share = m_k * 2 * (2 * ROW + 8) + m_n * (3 * ROW + 8)
                    total += G * (S * ROW + 4 * nk) + share
                    dom.append((share, G * cache.budget * (4 * ROW + 16)))
                st["n_kept"] = min(nk + S, cache.budget)

        with torch.cuda.stream(cache.stream):
            plan.run(hook)
        torch.cuda.synchronize()
    return total, dom


def hold(torch, stream, n_calls):
    """Keep `stream` busy (a spin kernel, about 30 us per call to come, outside
    any timed interval) so that the host has enqueued the calls before the GPU
    reaches them: the events then time the GPU's work, not host gaps."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(int(min(max(n_calls, 30), 2000) * 30e-6 * 2.4e9))


def timed_steps(torch, wl, n, graph=None):
    """Milliseconds of each of n steps, from one event pair per step on the
    launch stream (other streams join it before each event).  Without
    snapshots the steps run back to back, one event between two steps; with
    snapshots every step has its own pair and the untimed restore runs
    between them."""
    ev = torch.cuda.Event
    s0, rest = wl.streams[0], wl.streams[1:]

    def mark():
        for s in rest:
            j = ev()
            j.record(s)
            s0.wait_event(j)
        e = ev(enable_timing=True)
        e.record(s0)
        for s in rest:
            s.wait_event(e)
        return e

    def one():
        with torch.cuda.stream(s0):
            if graph is not None:
                graph.replay()
            else:
                wl.step()

    if not wl.snapshots:
        hold(torch, s0, n * wl.calls_per_step)
        marks = [mark()]
        for _ in range(n):
            one()
            marks.append(mark())
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(marks, marks[1:])]
    out = []
    for _ in range(n):
        wl.restore()
        torch.cuda.synchronize()
        hold(torch, s0, wl.calls_per_step)
        a = mark()
        one()
        b = mark()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def kernel_times(torch, wl, steps):
    """Second timed pass, one plan at a time (input sets rotated as in the
    timed steps): an event pair on the plan's own stream around every library
    call."""
    per = {}
    ev = torch.cuda.Event
    for s in range(steps):
        wl.restore()
        torch.cuda.synchronize()
        for p in wl.plan_sets[s % len(wl.plan_sets)]:
            rec = []
            hold(torch, p.cache.stream, len(p.calls))

            def hook(i, name, when, p=p, rec=rec):
                e = ev(enable_timing=True)
                e.record(p.cache.stream)
                rec.append((name, when, e))

            p.run(hook)
            torch.cuda.synchronize()
            for k in range(0, len(rec), 2):
                (n0, w0, e0), (n1, w1, e1) = rec[k], rec[k + 1]
                assert w0 == "before" and w1 == "after" and n0 == n1
                per.setdefault(n0, []).append(e0.elapsed_time(e1))
    return per


# ----------------------------------------------------------------------------- oracle leg


def oracle_leg(wl, captured, timed_state, base_groups, min_seconds=10.0):
    """Everything the oracle does in this benchmark, on bytes copied back from
    the device: (1) parity -- for every plan set and cache, the oracle replays
    its selection and compaction on the GPU's scores of every call
    (lockstep) and must end in the GPU's state bit for bit, after the capture
    pass and (for the set the last timed step ran) after the timed steps; its
    own scores must lie within 1e-5 of the GPU's, relative to the norm (L2)
    or to sum_d |k_d f_d| (projection); (2) the CPU baseline -- the oracle's
    own run (its own fp64 scores) over the same input bytes of `base_groups`,
    timed (skipped when min_seconds is 0).  Returns (parity, cpu_baseline)."""
    import oracle
    cfg = wl.cfg
    bit_exact, n_calls, worst, states_compared = True, 0, 0.0, 0
    mismatches = []
    timed_set = wl.last_set
    for si, (per_cache, state_after) in captured.items():
        for ci, calls in enumerate(per_cache):
            (l0, l1), sc = wl.ranges[ci], wl.scorer_of[ci]
            loc = wl.local(l0, l1)
            if not loc:
                continue
            f = _sample_filters(wl, ci, loc)
            keep = sc.keep if sc.mode == "l2" else "high"
            lock = oracle.OracleCache(len(loc), cfg.D, cfg.dtype, cfg.budget, cfg.n_sink, cfg.recent, keep,
                                      sc.mode, f, sc.sign)
            if wl.prefill_host is not None:
                i0 = [wl.sample.index(g + l0 * wl.bh) for g in loc]
                lock.update(wl.prefill_host[0][i0], wl.prefill_host[1][i0], scores_in=wl.prefill_scores[ci])
            for K, V, s_gpu in calls:
                lock.update(K, V, scores_in=s_gpu)
                worst = max(worst, _score_error(K, cfg.dtype, sc.mode, f, sc.sign, s_gpu))
                n_calls += 1
            states = [("capture pass, input set %d" % si, state_after[ci])]
            if si == timed_set and timed_state is not None:
                states.append(("after the timed steps", timed_state[ci]))
            for what, st in states:
                ok = _same_state(st, lock)
                states_compared += 1
                bit_exact &= ok
                if not ok:
                    mismatches.append("%s, cache %d" % (what, ci))
    parity = {"groups": len(wl.sample), "of": cfg.G, "runs": len(cfg.scorers), "input_sets": len(captured),
              "calls_replayed": n_calls, "states_compared": states_compared, "bit_exact": bool(bit_exact),
              "scores_within_tol": bool(worst <= 1.0), "max_score_err_over_tol": round(worst, 4),
              "compared": "kept rows, K/V bytes, stored scores and positions of every sampled group, after the "
                          "capture pass and after the timed steps; the oracle's rules replayed on the GPU's scores"}
    if mismatches:
        parity["mismatches"] = mismatches[:8]
    cb = None
    if min_seconds > 0:
        cb = cpu_baseline(wl, _baseline_bytes(wl, captured[0][0], base_groups), min_seconds)
    return parity, cb


def _sample_filters(wl, ci, loc):
    """Projection filters [len(loc), D] of cache ci's sampled groups: the
    GPU's own (the planted directions per layer and head, or the frozen
    fallback estimate per group)."""
    import numpy as np
    c = wl.caches[ci]
    if c.mode != "proj":
        return None
    f = c.filters.reshape(c.score_shape.L, c.H, c.D).cpu().numpy()
    per_group = c.score_shape.L == c.L * c.B        # [L*B, H, D] (one per group) or [L, H, D]
    out = [f[(g // c.H) if per_group else (g // c.H) // c.B, g % c.H] for g in loc]
    return np.ascontiguousarray(np.stack(out), dtype=np.float32)


def _score_error(K, dtype, mode, f, sign, s_gpu):
    """Worst |s_gpu - s_oracle| / (1e-5 * scale) over the rows of one call."""
    import numpy as np

    import oracle
    from kv_cache_token_amd import synth
    ng, S, Dd = K.shape
    if mode == "l2":
        ref = oracle.score(K.reshape(ng * S, Dd), "l2", None, 1, dtype).reshape(ng, S).astype(np.float64)
        scale = ref
    else:
        ref = np.stack([oracle.score(K[i], mode, f[i], sign, dtype) for i in range(ng)]).astype(np.float64)
        scale = np.stack([np.abs(synth.bits_to_f32(K[i], dtype).astype(np.float64)) @ np.abs(f[i].astype(np.float64))
                          for i in range(ng)])
    err = np.abs(s_gpu.astype(np.float64) - ref)
    bound = 1e-5 * scale
    ratio = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
    return float(ratio.max()) if ratio.size else 0.0


def _same_state(st, lock):
    import numpy as np
    k, v, s, p = st
    n = p.shape[1]
    if not np.all(lock.n == n):
        return False
    return (np.array_equal(p, lock.pos[:, :n]) and np.array_equal(s.view(np.uint32), lock.s[:, :n].view(np.uint32))
            and np.array_equal(k, lock.k[:, :n]) and np.array_equal(v, lock.v[:, :n]))


def _baseline_bytes(wl, per_cache, base_groups):
    """The CPU baseline's input: the captured bytes of the baseline groups (in
    the first layer range; every scorer run reads the same blocks)."""
    split = len(wl.caches) // len(wl.cfg.scorers)
    l0, l1 = wl.ranges[0]
    loc = wl.local(l0, l1)
    want = set(base_groups)
    sel = [i for i, g in enumerate(loc) if g + l0 * wl.bh in want]
    pre = None
    if wl.prefill_host is not None:
        i0 = [wl.sample.index(loc[i] + l0 * wl.bh) for i in sel]
        pre = (wl.prefill_host[0][i0], wl.prefill_host[1][i0])
    filt = []
    for i in range(len(wl.cfg.scorers)):
        f = _sample_filters(wl, i * split, loc)
        filt.append(None if f is None else f[sel])
    return {"groups": [loc[i] + l0 * wl.bh for i in sel], "chunks": [(K[sel], V[sel]) for K, V, _ in per_cache[0]],
            "prefill": pre, "filters": filt}


def recipe_bytes(cfg, n_groups):
    """The CPU baseline's input drawn from the seeded host recipe (numpy), for
    runs without a GPU."""
    import numpy as np

    from kv_cache_token_amd import synth
    from oracle import calib
    sample = synth.sample_groups(cfg, n_groups)
    if cfg.cid == 3:
        pre = synth.batch_chunk(cfg, sample, 0)
        dec = [synth.decode_block(cfg, g) for g in sample]
        chunks = [(np.stack([d[0][t:t + 1] for d in dec]), np.stack([d[1][t:t + 1] for d in dec]))
                  for t in range(256)]
    else:
        pre = None
        chunks = [synth.batch_chunk(cfg, sample, c) for c in range(len(cfg.chunks))]
    filt = []
    for sc in cfg.scorers:
        if sc.filt == "mu":
            f_lh = synth.filters_mu(cfg)
            filt.append(np.stack([f_lh[cfg.group_lbh(g)[0], cfg.group_lbh(g)[2]] for g in sample]))
        elif sc.filt == "keysvd":
            k0 = synth.bits_to_f32(chunks[0][0][:, :cfg.calib_tokens], cfg.dtype).astype(np.float64)
            filt.append(np.stack([calib.estimate_filter_dir(k0[i]) for i in range(len(sample))]).astype(np.float32))
        else:
            filt.append(None)
    return {"groups": sample, "chunks": chunks, "prefill": pre, "filters": filt}


def cpu_baseline(wl, inputs, min_seconds=10.0):
    """The oracle as it stands (its own fp64 scores), on `inputs` (the bytes
    of a sample of groups: from the device, or recipe_bytes), every run of the
    step, repeated from the same starting state until at least min_seconds of
    oracle time have run."""
    import oracle
    cfg = wl.cfg
    ns = len(inputs["groups"])
    caches = []
    for sc, f in zip(cfg.scorers, inputs["filters"]):
        keep = sc.keep if sc.mode == "l2" else "high"
        oc = oracle.OracleCache(ns, cfg.D, cfg.dtype, cfg.budget, cfg.n_sink, cfg.recent, keep, sc.mode, f, sc.sign)
        if inputs["prefill"] is not None:
            oc.update(*inputs["prefill"])      # the decode step starts from a full cache (untimed)
        caches.append(oc)
    chunks = inputs["chunks"]

    def run(seconds):
        t, reps = 0.0, 0
        while reps == 0 or (t < seconds and reps < 10000):
            fresh = [oc.copy() for oc in caches]
            t0 = time.perf_counter()
            for oc in fresh:
                for K, V in chunks:
                    oc.update(K, V)
            t += time.perf_counter() - t0
            reps += 1
        return reps * wl.tokens_per_step * ns / cfg.G / t, reps, t   # workload-equivalent tokens/s

    threads = oracle.num_threads()
    rate, reps, t = run(min_seconds)
    oracle.set_num_threads(1)
    rate1, _, _ = run(min_seconds / 4)
    oracle.set_num_threads(threads)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d groups, every run of the step, %d repetitions (%.1f s of oracle time)" % (
                ns, cfg.G, reps, t),
            "value_1_thread": round(rate1, 1), "cpu_model": model, "host_cpus": os.cpu_count()}


def copy_ceiling(torch, stream):
    """Device-to-device copy rate of the library's own row copy (the
    passthrough append into a separate buffer): 2 x 256 MiB of bf16 rows read
    and written, plus 4 B of position per row; GB/s."""
    from kv_cache_token_amd import api
    G, S = 1024, 1024
    shape = api.make_shape(G, 1, 1, "bf16")
    with torch.cuda.stream(stream):
        src_k = torch.empty((G, S, D), dtype=torch.bfloat16, device="cuda")
        src_v = torch.empty_like(src_k)
        dst_k, dst_v = torch.empty_like(src_k), torch.empty_like(src_k)
        pos = torch.empty((G, S), dtype=torch.int32, device="cuda")
    fn = lambda: api.kv_passthrough_append(None, None, 0, 0, src_k, src_v, S, shape, dst_k, dst_v, pos, S,  # noqa: E731
                                           stream)
    event_times(torch, stream, fn, 3)
    ms = event_times(torch, stream, fn, 10)
    return round((4 * src_k.numel() * 2 + pos.numel() * 4) / (ms * 1e-3) / 1e9, 1)


def per_layer_ms(torch, wl, steps):
    """Secondary number: the same step with one launch sequence per layer (a
    cache of B x H groups per layer) instead of all layers in each launch."""
    from kv_cache_token_amd.cache import EvictingCache
    cfg, st = wl.cfg, wl.streams[0]
    bh = cfg.B * cfg.H
    plans = []
    for sc in cfg.scorers:
        keep = sc.keep if sc.mode == "l2" else "high"
        for l in range(cfg.L):
            f = wl.f_mu[l:l + 1] if sc.filt == "mu" else None
            c = EvictingCache(1, cfg.B, cfg.H, cfg.budget, cfg.n_sink, cfg.recent, keep, sc.mode, f, sc.sign,
                              cfg.dtype, stream=st, head_dim=cfg.D)
            plans.append(c.plan([(k[l * bh:(l + 1) * bh], v[l * bh:(l + 1) * bh]) for k, v in wl.blocks]))
    run = lambda: [p.run() for p in plans]  # noqa: E731
    n_calls = sum(len(p.calls) for p in plans)
    event_times(torch, st, run, 1, n_calls)
    return round(event_times(torch, st, run, steps, n_calls), 4)


def event_times(torch, stream, fn, n, calls_per_fn=1):
    """Mean milliseconds of fn() over n launches, from HIP events on `stream`."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    hold(torch, stream, n * calls_per_fn)
    with torch.cuda.stream(stream):
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / n


def fallback_estimate_time(torch, wl):
    """Device time of the key-SVD fallback estimate of the c5 workload (all
    groups, the first calib_tokens keys of the first chunk)."""
    from kv_cache_token_amd import api
    cfg, st = wl.cfg, wl.streams[0]
    k0 = wl.blocks[0][0]
    f = torch.empty((cfg.G, cfg.D), dtype=torch.float32, device="cuda")
    status = torch.empty(cfg.G, dtype=torch.int32, device="cuda")
    fn = lambda: api.qf_filters_from_keys_device(k0, cfg.G, cfg.calib_tokens, k0.shape[1], f, status,  # noqa: E731
                                                 stream=st)
    event_times(torch, st, fn, 2)
    ms = event_times(torch, st, fn, 10)
    assert int(status.max()) == 0
    return {"groups": cfg.G, "keys_per_group": cfg.calib_tokens, "mean_us": round(ms * 1e3, 1)}


def bench_qcal(torch, args):
    """The query-SVD calibration at the pages' scale, on the device."""
    from kv_cache_token_amd import api, synth
    L, Hq, Hkv, N = 28, 24, 8, 3000
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        q = synth.query_acts_device(L, Hq, Hkv, N, D, seed=1)
        out = torch.empty((L, Hkv, D), dtype=torch.float32, device="cuda")
        status = torch.empty((L, Hkv), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    fn = lambda: api.qf_filters_from_queries_device(q, Hkv, out, status, stream=st)  # noqa: E731
    if args.warmup:
        event_times(torch, st, fn, args.warmup)
    ms = event_times(torch, st, fn, args.steps)
    assert int(status.max()) == 0
    # the Gram matrices: D (D + 1) / 2 distinct entries of a symmetric D x D
    # matrix, 2 N flops each (power iteration and squarings not counted)
    flops = float(N * D * (D + 1) * Hq * L)
    achieved = flops / (ms * 1e-3) / 1e12
    out_line = {
        "metric": "query-SVD calibration query heads/sec (fp64 Gram + power iteration + GQA averaging)",
        "value": round(Hq * L / (ms * 1e-3), 1), "unit": "query heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64",
        "data": "synthetic (seeded, HBM-resident; rows drift*mu_h + N(0,0.25), heads of a KV group leaning together)",
        "config": {"workload": DESCRIPTIONS["qcal"], "device": torch.cuda.get_device_name(0)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP64_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP64_TFLOPS, 4), "traffic": None,
                     "kernel": "top_direction_kernel (symmetric Gram flops only)",
                     "algorithmic_flops_per_launch": int(flops), "mean_launch_us": round(ms * 1e3, 1)},
    }
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle import calib
        qh = synth.query_acts(1, Hq, Hkv, N, D, seed=1, dtype="bf16")[0]
        x = synth.bf16_bits_to_f32(qh).astype(np.float64)
        t0 = time.perf_counter()
        calib.average_gqa_filters(calib.compute_qfilters(x), Hkv)
        sec = time.perf_counter() - t0
        out_line["cpu_baseline"] = {"value": round(Hq / sec, 1), "unit": "query heads/s",
                                    "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                                    "kind": "oracle", "sample": "one layer (24 query heads x 3000 x 128), numpy SVD"}
    print(json.dumps(out_line), flush=True)


def variant_config(args):
    """The workload's config with the variant options applied, and a text
    naming them ("" when none is given)."""
    import dataclasses
    from kv_cache_token_amd import synth
    opts = {k: getattr(args, k, None) for k in ("dtype", "head_dim", "budget", "chunk", "tokens", "layers")
            if getattr(args, k, None) is not None}
    if args.workload == "qcal" and not opts:
        return None, ""
    if opts and args.workload not in ("c2", "c4", "c5"):
        log("size variants apply to the prefill workloads c2, c4 and c5")
        sys.exit(2)
    cfg = synth.CONFIGS[int(args.workload[1:])]
    if not opts:
        return cfg, ""
    chunk = opts.get("chunk", cfg.chunks[0])
    tokens = opts.get("tokens", cfg.tokens)
    if tokens % chunk or chunk < 1:
        log("--tokens must be a positive multiple of --chunk")
        sys.exit(2)
    head_dim = opts.get("head_dim", cfg.D)
    if head_dim == 256 and any(sc.filt == "keysvd" for sc in cfg.scorers):
        log("the key-SVD fallback estimates filters on the device for head dims 64 and 128 only")
        sys.exit(2)
    layers = opts.get("layers", cfg.L)
    if layers < 1:
        log("--layers must be positive")
        sys.exit(2)
    cfg = dataclasses.replace(cfg, dtype=opts.get("dtype", cfg.dtype), D=head_dim, L=layers,
                              budget=opts.get("budget", cfg.budget), chunks=(chunk,) * (tokens // chunk))
    text = "variant: %d layer%s, %s K/V, head_dim %d, budget %d, %d tokens per run in %d-token chunks" % (
        cfg.L, "" if cfg.L == 1 else "s", cfg.dtype, cfg.D, cfg.budget, tokens, chunk)
    return cfg, text


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c4", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2, 4),
                    help="streams the step's independent caches are spread over (2: the two scorer runs of c4 "
                         "side by side)")
    ap.add_argument("--split", type=int, default=1,
                    help="divide each run's groups by layer into this many independent caches")
    ap.add_argument("--cpu-groups", type=int, default=32, help="groups in the oracle's timed sample")
    ap.add_argument("--parity-groups", type=int, default=0,
                    help="groups the oracle checks bit for bit (0: 224, or all groups if fewer; 64 for c5)")
    ap.add_argument("--no-parity", action="store_true", help="skip the capture pass and the oracle's parity check")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle's sample until this much oracle time has run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the secondary measurements (per-layer launches, device copy rate), e.g. under a "
                         "kernel trace whose per-kernel averages should cover the step's own launches only")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as one captured HIP graph (workloads without snapshots, one stream)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (reference for byte counters)")
    vg = ap.add_argument_group("variants of a prefill workload (c2, c4, c5): the same recipe with other sizes")
    vg.add_argument("--dtype", choices=("bf16", "f16", "f32"), help="K/V element type")
    vg.add_argument("--head-dim", type=int, choices=(64, 128, 256))
    vg.add_argument("--budget", type=int, help="rows kept per group")
    vg.add_argument("--chunk", type=int, help="tokens per call")
    vg.add_argument("--tokens", type=int, help="tokens per run (a multiple of the chunk)")
    vg.add_argument("--layers", type=int, help="layers (each with the workload's KV heads)")
    args = ap.parse_args()
    if args.gpus != 1:
        log("bench.py measures one GPU: the library has no multi-GPU path (each GPU would run the same "
            "step on its own groups); run with --gpus 1")
        sys.exit(2)
    cfg, variant = variant_config(args)

    import torch
    from kv_cache_token_amd import _lib
    _lib.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "qcal":
        bench_qcal(torch, args)
        return
    from kv_cache_token_amd import synth
    dev_name = torch.cuda.get_device_name(0)
    streams = [torch.cuda.Stream() for _ in range(args.streams)]
    base_groups = synth.sample_groups(cfg, args.cpu_groups)
    n_par = args.parity_groups or (64 if args.workload == "c5" else min(224, cfg.G))
    sample = [] if args.no_parity else sorted(set(synth.sample_groups(cfg, n_par)) | set(base_groups))
    wl = Workload(torch, args.workload, streams, args.split, cfg, sample=sample)
    cfg = wl.cfg
    log("workload %s ready on %s: %d groups, %d calls per run" % (args.workload, dev_name, cfg.G, len(wl.blocks)))

    if args.copy_calibration:
        with torch.cuda.stream(streams[0]):
            src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
            dst = torch.empty_like(src)
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step_bytes, dom_bytes = algorithmic_bytes(torch, wl)
    log("algorithmic bytes per step: %.3f GB" % (step_bytes / 1e9))
    captured = None
    if sample:
        captured = capture_pass(torch, wl)
        log("capture pass: %d groups' bytes and scores copied back" % len(sample))
    graph = None
    if args.graph:
        if wl.snapshots or len(streams) > 1:
            log("--graph needs a workload without snapshots on one stream")
            sys.exit(2)
        with torch.cuda.stream(streams[0]):
            wl.step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=streams[0]):
            wl.step()
        torch.cuda.synchronize()
    if args.warmup:
        timed_steps(torch, wl, args.warmup, graph)
    step_ms = timed_steps(torch, wl, args.steps, graph)
    ms_per_step = float(np.median(step_ms))
    timed_state = sampled_state(wl) if sample else None

    per = kernel_times(torch, wl, args.steps)
    breakdown = {n: {"launches_per_step": len(v) // args.steps, "mean_us": round(1e3 * sum(v) / len(v), 2)}
                 for n, v in per.items()}
    chunk_sizes = {k.shape[1] for k, _ in wl.blocks}
    if "qf_score_keys" in breakdown and len(chunk_sizes) == 1:
        # scoring reads each incoming row once and writes its score
        sb = cfg.G // args.split * chunk_sizes.pop() * (wl.row + 4)
        e = breakdown["qf_score_keys"]
        e["algorithmic_bytes_per_launch"] = sb
        e["GBps"] = round(sb / (e["mean_us"] * 1e-6) / 1e9, 1)
    dom_ms = per[wl.dominant]
    if wl.dominant == "kv_compact_gather":
        # evicting launches only: the leading calls of each run that only append are left out
        calls_per_run = len(dom_ms) // (args.steps * len(wl.plans))
        n_append = calls_per_run - len(dom_bytes) // len(wl.plans)
        dom_ms = [x for n, x in enumerate(dom_ms) if n % calls_per_run >= n_append]
    mean_ms = sum(dom_ms) / len(dom_ms)
    bytes_per_launch = sum(a for a, _ in dom_bytes) / len(dom_bytes)
    impl_per_launch = sum(b for _, b in dom_bytes) / len(dom_bytes)
    achieved = bytes_per_launch / (mean_ms * 1e-3) / 1e9
    sha = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]
    mt = None if variant else MEASURED_TRAFFIC.get(args.workload)
    traffic = mt["bytes_per_launch"] if mt and sha == mt["kernel_src_sha256_16"] else None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic, "traffic_unit": "bytes/launch",
            "kernel": wl.dominant + (" (evicting calls)" if wl.dominant == "kv_compact_gather" else ""),
            "launches": len(dom_ms), "mean_launch_us": round(mean_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": int(bytes_per_launch),
            "kernel_bytes_per_launch": int(impl_per_launch),
            "kernel_GBps": round(impl_per_launch / (mean_ms * 1e-3) / 1e9, 1),
            "traffic_over_algorithmic": None if traffic is None else round(traffic / bytes_per_launch, 4)}
    value = wl.tokens_per_step / (ms_per_step * 1e-3)
    step_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": "evicted-cache tokens/sec (score+select+compact), achieved HBM GB/s vs peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "ms_per_step_stats": {"median": round(ms_per_step, 4), "mean": round(float(np.mean(step_ms)), 4),
                              "min": round(float(np.min(step_ms)), 4), "max": round(float(np.max(step_ms)), 4),
                              "steps_timed": len(step_ms)},
        "dtype": cfg.dtype,
        "data": "synthetic (seeded, HBM-resident; keys %s, V ~ N(0,1))" % {
            "aniso": "drift*mu + N(0,0.25)", "lognorm": "r*u, ln r ~ N(0,0.25)", "gauss": "N(0,1)"}[cfg.keys],
        "config": {"workload": DESCRIPTIONS[args.workload] + ("; " + variant if variant else ""), "groups": cfg.G,
                   "tokens_per_step": wl.tokens_per_step, "runs_per_step": len(wl.plans),
                   "budget": cfg.budget, "streams": args.streams, "split": args.split, "graph": bool(graph),
                   "input_sets": len(wl.plan_sets), "device": dev_name},
        "head_tokens_per_s": round(value * cfg.L * cfg.H, 1),
        "step_algorithmic_GBps": round(step_gbps, 1), "step_frac_of_peak": round(step_gbps / PEAK_HBM_GBPS, 4),
        "step_algorithmic_bytes": int(step_bytes),
        "device_copy_GBps": None if args.no_extras else copy_ceiling(torch, streams[0]),
        "roofline": roof,
        "kernels": breakdown,
    }
    if args.workload == "c5":
        out["fallback_estimate"] = fallback_estimate_time(torch, wl)
    if args.workload in ("c2", "c4") and args.split == 1 and graph is None \
            and not args.no_extras:
        out["per_layer_ms_per_step"] = per_layer_ms(torch, wl, max(1, args.steps // 4))
    parity = cb = None
    if sample:
        parity, cb = oracle_leg(wl, captured, timed_state, base_groups,
                                0.0 if args.no_cpu_baseline else args.cpu_seconds)
        out["parity"] = parity
    if cb is not None:
        cb["algorithmic_GBps"] = round(cb["value"] * step_bytes / wl.tokens_per_step / 1e9, 2)
        cb["gpu_speedup"] = round(value / cb["value"], 1)
        cb["inputs"] = "the same device bytes the GPU step read, copied back before timing"
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    if parity is not None and not (parity["bit_exact"] and parity["scores_within_tol"]):
        log("PARITY FAILURE: %s" % json.dumps(parity))
        sys.exit(1)


if __name__ == "__main__":
    main()
