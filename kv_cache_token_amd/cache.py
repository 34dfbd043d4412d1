"""EvictingCache: the per-model bounded KV cache driven by the C ABI.

It owns the device buffers (two cache buffer sets used alternately when a block
evicts, a keep-index buffer and the incoming-score buffer), the kept-row count
and the true offset (tokens seen, Q-Filters page, "RoPE positions had to be
fixed first").  Each ``update`` is the query-free step of the pages
(Q-Filters page and L2Norm page, "How it works"): score the incoming rows,
select, compact -- or, when the block evicts nothing, score and append in one
pass; all arithmetic runs in the library's kernels on one stream.
A projection cache built without filters runs the key-SVD fallback's lifecycle
on the device (Q-Filters page, "How it works" step 2, "Key-SVD fallback"):
rows are held unscored below calib_tokens, and the crossing block freezes one
filter per group and runs the step over everything held.
"""
from __future__ import annotations

import numpy as np

from . import api

LAST_LEVEL_CACHE_BYTES = 256 << 20   # MI355X's last-level (Infinity) cache


class EvictingCache:
    """Bounded KV cache of L layers x B sequences x H KV heads (G = L*B*H groups).

    budget, n_sink, recent, keep: the step's parameters (the budget includes the
    sinks; keep is "low" or "high" for the L2 scorer, always "high" for
    projection).  mode "l2" or "proj"; filters [L, H, D] float32 for projection,
    or None with calib_tokens >= 2 for the key-SVD fallback (calib_keys
    "crossing": estimate from every key held when the crossing block arrives;
    "first": from the first calib_tokens keys).  dtype "bf16", "f16" or "f32";
    head_dim 64, 128 or 256.  `stream` is the HIP stream (torch stream or raw
    handle) every call is enqueued on; None uses torch's current stream."""

    def __init__(self, L: int, B: int, H: int, budget: int, n_sink: int = 4, recent: int = 0,
                 keep: str = "low", mode: str = "l2", filters=None, sign: int = 1, dtype: str = "bf16",
                 device="cuda", calib_tokens: int = 0, stream=None, head_dim: int = 128,
                 calib_keys: str = "crossing", calib_max_iter: int = 20000):
        import torch
        self.L, self.B, self.H, self.G = L, B, H, L * B * H
        self.budget, self.n_sink, self.recent = budget, n_sink, recent
        self.mode, self.sign = mode, sign
        self.keep = "high" if mode == "proj" else keep
        self.D = head_dim
        self.dtype_name = {"bf16": "bf16", "f16": "f16", "f32": "f32"}.get(dtype, dtype)
        self.shape = api.make_shape(L, B, H, dtype, head_dim)
        self.params = api.make_params(budget, n_sink, recent, self.keep)
        self.calib_tokens = calib_tokens
        self.calib_keys = calib_keys
        self.calib_max_iter = calib_max_iter
        self.stream = stream
        self.device = torch.device(device)
        if calib_keys not in ("crossing", "first"):
            raise ValueError("calib_keys must be 'crossing' or 'first'")
        if mode == "proj" and filters is None:
            if calib_tokens < 2:
                raise ValueError("projection needs filters or calib_tokens >= 2 (key-SVD fallback)")
            if head_dim not in (64, 128):
                raise ValueError("the key-SVD fallback estimates filters on the device for head dims 64 "
                                 "and 128; pass filters for head dim %d" % head_dim)
        if mode not in ("l2", "proj"):
            raise ValueError("mode must be 'l2' or 'proj'")
        if n_sink + recent >= budget:
            raise ValueError("n_sink + recent must be below budget")
        if mode == "proj" and sign not in (1, -1):
            raise ValueError("sign must be +1 or -1")
        td = api.torch_dtype(self.shape.dtype)
        G = self.G

        def bufset():
            return (torch.empty((G, budget, head_dim), dtype=td, device=self.device),
                    torch.empty((G, budget, head_dim), dtype=td, device=self.device),
                    torch.empty((G, budget), dtype=torch.float32, device=self.device),
                    torch.empty((G, budget), dtype=torch.int32, device=self.device))

        self._bufs = [bufset(), bufset()]
        self._cur = 0
        self.keep_idx = torch.empty((G, budget), dtype=torch.int32, device=self.device)
        self._s_new = torch.empty((G, 1), dtype=torch.float32, device=self.device)
        self.score_shape = self.shape
        self.filters = None
        if filters is not None:
            self.set_filters(filters)
        self.n_kept = 0
        self.tokens_seen = 0
        self._held = None          # pre-calibration rows (k, v, pos) [G, calib_tokens - 1, *]
        self.calib_status = None   # [G] int32 of the last fallback estimate

    # -- filters -----------------------------------------------------------
    def set_filters(self, filters, per_group: bool = False) -> None:
        """Freeze the projection filters: [L, H, D] (per layer and KV head) or,
        with per_group, [G, D] (one per (layer, batch, head) group)."""
        import torch
        f = torch.as_tensor(np.asarray(filters, dtype=np.float32) if not isinstance(filters, torch.Tensor)
                            else filters, dtype=torch.float32)
        if per_group:
            f = f.reshape(self.L * self.B, self.H, self.D)
            self.score_shape = api.make_shape(self.L * self.B, 1, self.H, self.shape.dtype, self.D)
        else:
            f = f.reshape(self.L, self.H, self.D)
            self.score_shape = self.shape
        self.filters = f.to(self.device).contiguous()

    @property
    def calibrating(self) -> bool:
        """True while the key-SVD fallback filter has not been frozen yet."""
        return self.mode == "proj" and self.filters is None

    def _passthrough(self, k_new, v_new, S: int, prepare: bool):
        """Hold the block unscored (Q-Filters page, "How it works" step 2: with
        no filter there is no eviction, even over budget)."""
        import torch
        cap = self.calib_tokens - 1
        if self._held is None:
            td = api.torch_dtype(self.shape.dtype)
            self._held = (torch.empty((self.G, cap, self.D), dtype=td, device=self.device),
                          torch.empty((self.G, cap, self.D), dtype=td, device=self.device),
                          torch.empty((self.G, cap), dtype=torch.int32, device=self.device))
        hk, hv, hp = self._held
        call = api.kv_passthrough_append(hk, hv, self.n_kept, cap, k_new, v_new, S, self.shape, hk, hv, hp, cap,
                                         self.stream, prepare=prepare)
        self.n_kept += S
        self.tokens_seen += S
        return [call] if prepare else []

    def _crossing(self, k_new, v_new, S: int, prepare: bool):
        """The block that brings the tokens seen to calib_tokens: estimate every
        group's filter from the keys held so far plus this block (all of them,
        or with calib_keys="first" the first calib_tokens), freeze it, then run
        the step over the whole concatenation from an empty cache, so that every
        held row is scored with the frozen filter (Q-Filters page, "How it
        works" step 2, "Key-SVD fallback", "Path dependence")."""
        import torch
        calls = []
        n_held, n_total = self.n_kept, self.n_kept + S
        if n_held == 0:
            bk, bv, extra = k_new, v_new, ()
        else:
            td = api.torch_dtype(self.shape.dtype)
            bk = torch.empty((self.G, n_total, self.D), dtype=td, device=self.device)
            bv = torch.empty_like(bk)
            bp = torch.empty((self.G, n_total), dtype=torch.int32, device=self.device)
            hk, hv, _ = self._held
            extra = self._held + (bp,)
            calls.append(api.kv_passthrough_append(hk, hv, n_held, self.calib_tokens - 1, k_new, v_new, S,
                                                   self.shape, bk, bv, bp, n_total, self.stream, prepare=prepare))
        n_calib = n_total if self.calib_keys == "crossing" else self.calib_tokens
        f = torch.empty((self.G, self.D), dtype=torch.float32, device=self.device)
        self.calib_status = torch.empty(self.G, dtype=torch.int32, device=self.device)
        calls.append(api.qf_filters_from_keys_device(bk, self.G, n_calib, n_total, f, self.calib_status,
                                                     self.calib_max_iter, self.stream, prepare=prepare))
        self.set_filters(f, per_group=True)
        if not prepare:
            self.check_calibration()
        self._held = None
        self.n_kept, self.tokens_seen = 0, 0
        more, refs = self._step(bk, bv, prepare)
        return calls + more, (bk, bv, f, self.calib_status) + extra + tuple(refs)

    def check_calibration(self) -> None:
        """Wait for the last fallback estimate and raise if a group has no
        dominant key direction (status 1: top two eigenvalues not separated;
        2: its centred keys are all zero)."""
        import torch
        if self.calib_status is None:
            return
        torch.cuda.synchronize(self.device)
        st = self.calib_status.cpu().numpy()
        bad = np.flatnonzero(st)
        if bad.size:
            raise RuntimeError("key-SVD fallback: %d group(s) have no dominant key direction (first: group %d, "
                               "status %d)" % (bad.size, int(bad[0]), int(st[bad[0]])))

    # -- state -------------------------------------------------------------
    @property
    def offset(self) -> int:
        """Absolute tokens absorbed (the position the next token will get)."""
        return self.tokens_seen

    def buffers(self):
        return self._bufs[self._cur]

    def kept(self):
        """Views (k, v, s, pos) of the kept rows; before the fallback filter is
        frozen the held rows, with s None (they are not scored yet)."""
        n = self.n_kept
        if self.calibrating:
            if self._held is None:
                k, v, _, p = self._bufs[self._cur]
                return k[:, :0], v[:, :0], None, p[:, :0]
            hk, hv, hp = self._held
            return hk[:, :n], hv[:, :n], None, hp[:, :n]
        k, v, s, p = self._bufs[self._cur]
        return k[:, :n], v[:, :n], s[:, :n], p[:, :n]

    def last_scores(self):
        """Scores [G, S] the last update computed for its incoming rows."""
        return self._s_new

    def reset(self, keep_filters: bool = False) -> None:
        """Empty the cache.  Fallback filters (estimated from the stream's first
        keys) are forgotten unless keep_filters is set."""
        self.n_kept = 0
        self.tokens_seen = 0
        self._held = None
        if not keep_filters and self.mode == "proj" and self.calib_tokens > 0 and self.score_shape is not self.shape:
            self.filters = None

    def stats(self) -> dict:
        return api.kvx_stats(self.shape, self.tokens_seen, self.n_kept, self.mode)

    # -- checkpoint ----------------------------------------------------------
    STATE_VERSION = 1

    def _config(self) -> dict:
        return {"L": self.L, "B": self.B, "H": self.H, "D": self.D, "dtype": self.dtype_name, "budget": self.budget,
                "n_sink": self.n_sink, "recent": self.recent, "keep": self.keep, "mode": self.mode,
                "sign": self.sign, "calib_tokens": self.calib_tokens, "calib_keys": self.calib_keys}

    def save_state(self, path: str) -> None:
        """Write the cache's state to an uncompressed .npz holding no pickled
        objects: the kept rows of every group (K and V as their stored bytes,
        stored scores, positions), the kept count and the true offset, the
        frozen filters, and, while a key-SVD fallback cache is still
        calibrating, the rows it holds.  A cache built with the same parameters
        resumes the stream from it (load_state).  Waits for the device.
        (Q-Filters page, "Calibrated": only the filters are saved there; the
        cache state itself is a convenience of this library.)"""
        import json
        import torch
        torch.cuda.synchronize(self.device)
        meta = dict(self._config(), version=self.STATE_VERSION, n_kept=self.n_kept, tokens_seen=self.tokens_seen,
                    calibrating=self.calibrating, per_group_filters=self.score_shape is not self.shape)
        k, v, sc, p = self.kept()
        out = {"meta": np.array(json.dumps(meta)), "k": _host_bits(k), "v": _host_bits(v),
               "pos": p.cpu().numpy()}
        if sc is not None:
            out["s"] = sc.cpu().numpy()
        if self.filters is not None:
            out["filters"] = self.filters.cpu().numpy()
        with open(path, "wb") as f:
            np.savez(f, **out)

    def load_state(self, path: str) -> None:
        """Resume from a file written by save_state; the cache's parameters
        (shape, element type, budget, protection, scorer) must match the
        saved ones (ValueError otherwise).  The kept rows land in the first
        buffer set; the call returns once they are on the device."""
        import json
        import torch
        with np.load(path, allow_pickle=False) as z:
            meta = json.loads(str(z["meta"]))
            arrays = {name: z[name] for name in z.files if name != "meta"}
        if meta.get("version") != self.STATE_VERSION:
            raise ValueError("cache state version %r, expected %d" % (meta.get("version"), self.STATE_VERSION))
        want = self._config()
        diff = {k: (meta.get(k), v) for k, v in want.items() if meta.get(k) != v}
        if diff:
            raise ValueError("cache state was saved with other parameters: %s" % ", ".join(
                "%s %r (this cache: %r)" % (k, a, b) for k, (a, b) in sorted(diff.items())))
        n = int(meta["n_kept"])
        self._check_state_arrays(meta, arrays)
        td = api.torch_dtype(self.shape.dtype)
        with torch.cuda.device(self.device):
            if "filters" in arrays:
                self.set_filters(torch.from_numpy(arrays["filters"]), per_group=bool(meta["per_group_filters"]))
            else:
                self.filters, self.score_shape = None, self.shape
            k = _device_rows(arrays["k"], td, self.device)
            v = _device_rows(arrays["v"], td, self.device)
            p = torch.from_numpy(arrays["pos"]).to(self.device)
            if meta["calibrating"]:
                cap = self.calib_tokens - 1
                self._held = (torch.empty((self.G, cap, self.D), dtype=td, device=self.device),
                              torch.empty((self.G, cap, self.D), dtype=td, device=self.device),
                              torch.empty((self.G, cap), dtype=torch.int32, device=self.device))
                for dst, src in zip(self._held, (k, v, p)):
                    dst[:, :n].copy_(src)
            else:
                self._held = None
                self._cur = 0
                bk, bv, bs, bp = self._bufs[0]
                bk[:, :n].copy_(k)
                bv[:, :n].copy_(v)
                bs[:, :n].copy_(torch.from_numpy(arrays["s"]).to(self.device))
                bp[:, :n].copy_(p)
            torch.cuda.synchronize(self.device)   # the copies are done before any stream reads them
        self.n_kept, self.tokens_seen = n, int(meta["tokens_seen"])
        self.calib_status = None

    def _check_state_arrays(self, meta: dict, arrays: dict) -> None:
        """Every array of a state file has the shape and element type the
        cache's parameters and the saved counts give (ValueError otherwise),
        so that nothing is broadcast or truncated on the way to the device."""
        n, seen, calibrating = meta.get("n_kept"), meta.get("tokens_seen"), meta.get("calibrating")
        cap = self.calib_tokens - 1 if calibrating else self.budget
        if not (isinstance(n, int) and isinstance(seen, int) and 0 <= n <= cap and n <= seen):
            raise ValueError("cache state: n_kept %r / tokens_seen %r do not fit this cache (at most %d rows)"
                             % (n, seen, cap))
        if calibrating and not (self.mode == "proj" and self.calib_tokens > 0):
            raise ValueError("cache state holds unscored rows, but this cache does not calibrate")
        row = np.dtype(np.float32 if self.dtype_name == "f32" else np.uint16)
        want = {"k": ((self.G, n, self.D), row), "v": ((self.G, n, self.D), row),
                "pos": ((self.G, n), np.dtype(np.int32))}
        if not calibrating:
            want["s"] = ((self.G, n), np.dtype(np.float32))
        if "filters" in arrays and self.mode == "proj":
            rows = self.L * self.B if meta.get("per_group_filters") else self.L
            want["filters"] = ((rows, self.H, self.D), np.dtype(np.float32))
        extra = sorted(set(arrays) - set(want))
        if extra:
            raise ValueError("cache state: unexpected arrays %s" % ", ".join(extra))
        for name, (shape, dt) in want.items():
            a = arrays.get(name)
            if a is None or a.shape != shape or a.dtype != dt:
                raise ValueError("cache state: %s is %s, expected %s %s" % (
                    name, "missing" if a is None else "%s %s" % (a.dtype, a.shape), dt, shape))

    # -- the step ----------------------------------------------------------
    def _workspace(self, n_kept: int, S: int):
        """Device workspace the selection needs for this call (None when it
        selects on chip); grown on demand and reused."""
        import torch
        need = api.kv_evict_workspace_size(self.shape, n_kept, S, self.params)
        if need == 0:
            return None
        if getattr(self, "_ws", None) is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self._ws

    def _cache_keys(self, S: int) -> bool:
        """Whether scoring should leave the block's keys in the last-level
        cache for the compaction of an evicting call: they must fit it, and the
        compaction must be expected to re-read at least a quarter of them
        (about budget / n_total of them)."""
        row = self.D * (4 if self.dtype_name == "f32" else 2)
        if self.G * S * row > 0.9 * LAST_LEVEL_CACHE_BYTES:
            return False
        return 4 * self.budget >= self.n_kept + S

    def _scores(self, S: int):
        import torch
        if self._s_new.shape[1] != S:
            self._s_new = torch.empty((self.G, max(S, 1)), dtype=torch.float32, device=self.device)
        return self._s_new

    def update(self, k_new, v_new) -> None:
        """Absorb one block: k_new, v_new [G, S, D] (or [L, B, H, S, D])."""
        self._step(k_new, v_new, prepare=False)

    def update_and_fetch(self, k_new, v_new):
        """The pages' per-block call (Q-Filters page, "Usage"): absorb the block
        and return the kept rows' (K, V) views [G, n, D] in temporal order;
        `offset` is then the true position of the next token."""
        self.update(k_new, v_new)
        k, v, _, _ = self.kept()
        return k, v

    def _step(self, k_new, v_new, prepare: bool):
        S = k_new.shape[-2]
        k_new = k_new.contiguous().reshape(self.G, S, self.D)
        v_new = v_new.contiguous().reshape(self.G, S, self.D)
        calls = []
        if S == 0:
            return calls, (k_new, v_new)
        if self.calibrating:
            if self.tokens_seen + S < self.calib_tokens:
                calls = self._passthrough(k_new, v_new, S, prepare)
                return calls, (k_new, v_new) + self._held
            return self._crossing(k_new, v_new, S, prepare)
        s_new = self._scores(S)
        k, v, s, p = self._bufs[self._cur]
        nk, pos_base = self.n_kept, self.tokens_seen
        ws = None
        if S > 1 and nk + S <= self.budget:
            # nothing is evicted: score and append in one pass (keys read once)
            calls.append(api.kv_score_append(k_new, v_new, self.score_shape, S, self.mode, self.filters, self.sign,
                                             pos_base, nk, self.params, k, v, s, p, s_new, self.stream,
                                             prepare=prepare))
            self.n_kept = nk + S
            self.tokens_seen += S
            return calls, (k_new, v_new, s_new, ws, self.filters)
        calls.append(api.qf_score_keys(k_new, self.score_shape, S, self.mode, self.filters, self.sign, s_new,
                                       self.stream, prepare=prepare, cache_keys=self._cache_keys(S)))
        if S == 1:
            calls.append(api.kv_evict_one_inplace(k, v, s, p, k_new, v_new, s_new, pos_base, self.shape, nk,
                                                  self.params, self.stream, prepare=prepare))
        else:
            ws = self._workspace(nk, S)
            calls.append(api.kv_evict_topk(s, s_new, self.shape, nk, S, self.params, self.keep_idx, ws,
                                           self.stream, prepare=prepare))
            ko, vo, so, po = self._bufs[1 - self._cur]
            calls.append(api.kv_compact_gather(k, v, s, p, k_new, v_new, s_new, pos_base, self.keep_idx,
                                               self.shape, nk, S, self.params, ko, vo, so, po, self.stream,
                                               prepare=prepare))
            self._cur = 1 - self._cur
        self.n_kept = min(nk + S, self.budget)
        self.tokens_seen += S
        # every tensor a prepared call points at: a later step may replace the
        # workspace, and set_filters the filters, while a plan still uses them
        return calls, (k_new, v_new, s_new, ws, self.filters)

    def plan(self, blocks, keep_state: bool = False) -> "StreamPlan":
        """Validate and record, once, the library calls that absorb `blocks`
        (a list of (K, V) device tensors) into an empty cache, or, with
        keep_state, into the cache as it stands (the caller then restores the
        buffers before each replay).  The plan replays the calls with no
        per-call marshalling (or inside a captured HIP graph) and keeps the
        tensors it points at alive (workspaces and filters included, even if
        a later call replaces the cache's own).  The cache's bookkeeping is left
        at the plan's starting state, and each run leaves it at the plan's final
        state.  A stream that starts a key-SVD fallback cache records the
        passthrough and the estimate as well; the filters are frozen to a
        buffer the plan writes when it runs, and the cache points at that
        buffer only once a run has been enqueued (StreamPlan.check reads the
        estimate's status)."""
        start = (self.n_kept, self.tokens_seen, self._cur) if keep_state else (0, 0, 0)
        start_aux = self._aux_state(None if not keep_state else self._held)
        self.n_kept, self.tokens_seen, self._cur = start
        self._set_aux(start_aux)
        calls, keep = [], []
        for k, v in blocks:
            c, refs = self._step(k, v, prepare=True)
            calls += c
            keep.append(refs)
        final = (self.n_kept, self.tokens_seen, self._cur)
        final_aux = self._aux_state(self._held)
        keep.append(final_aux)
        self.n_kept, self.tokens_seen, self._cur = start
        self._set_aux(start_aux)
        return StreamPlan(self, calls, start, final, keep, start_aux, final_aux)

    def _aux_state(self, held):
        """What a plan's calls change besides the counters: the frozen filters
        (the fallback freezes them into a buffer the plan writes), the shape
        they are read with, the estimate's status and the held rows."""
        return (self.filters, self.score_shape, self.calib_status, held)

    def _set_aux(self, aux) -> None:
        self.filters, self.score_shape, self.calib_status, self._held = aux


def _host_bits(t) -> np.ndarray:
    """Host copy of K/V rows as their stored bytes (uint16 for 16-bit types)."""
    import torch
    t = t.detach().contiguous()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _device_rows(a: np.ndarray, td, device):
    """Device tensor of element type td from stored row bytes (_host_bits)."""
    import torch
    if a.dtype == np.float32:
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(td)


class StreamPlan:
    """Prepared library calls of a whole block stream (see EvictingCache.plan)."""

    def __init__(self, cache: EvictingCache, calls, start, final, keepalive, start_aux, final_aux):
        self.cache, self.calls, self.start, self.final, self._keep = cache, calls, start, final, keepalive
        self.start_aux, self.final_aux = start_aux, final_aux

    def check(self) -> None:
        """After run(): wait and raise if a fallback estimate the plan made failed."""
        self.cache.check_calibration()

    @property
    def names(self):
        return [f.__name__ for f, _ in self.calls]

    def run(self, hook=None) -> None:
        """Enqueue every call from the plan's starting state; hook(i, name, when)
        with when in ("before", "after") is called around each call."""
        c = self.cache
        c.n_kept, c.tokens_seen, c._cur = self.start
        c._set_aux(self.start_aux)
        for i, (f, args) in enumerate(self.calls):
            if hook:
                hook(i, f.__name__, "before")
            rc = f(*args)
            if rc != 0:
                from . import _lib
                _lib.check(f.__name__, rc)
            if hook:
                hook(i, f.__name__, "after")
        c.n_kept, c.tokens_seen, c._cur = self.final
        c._set_aux(self.final_aux)
