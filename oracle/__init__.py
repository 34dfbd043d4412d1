"""CPU oracle for the query-free KV-cache eviction step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s oracle leg (the
parity check of its own run and the CPU baseline, both on bytes copied back
from the device) import this package.  The product (``kv_cache_token_amd`` and its HIP library)
never imports it, and the two share no code: the only common input is the
seeded generator module ``kv_cache_token_amd.synth``, which holds none of the
method's arithmetic.

The eviction rules live in ``kvx_oracle.c`` (plain C, fp64 scoring, a plain sort
for the ranking); this module loads it with ctypes, building it with gcc if the
shared object is absent.  The calibration rules (query-SVD filter, GQA averaging,
key-SVD fallback) live in ``calib.py`` and use numpy's SVD; ``FallbackOracleCache``
composes the fallback estimate with the step in the lifecycle the Q-Filters page
describes (passthrough below calib_tokens, freeze at the crossing block).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
brute force, closed forms, an independent streaming implementation and the
invariants the pages state; see the docstrings there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

from . import calib  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvx_oracle.c")
_BUILT = os.path.join(_HERE, "libkvx_oracle.so")
# KVX_ORACLE_LIB names another build of the same source (the sanitizer build).
_LIB = os.environ.get("KVX_ORACLE_LIB") or _BUILT
_lib = None

MODE_L2, MODE_PROJ = 0, 1
DT_F32, DT_BF16, DT_F16 = 0, 1, 2
_DT = {"f32": DT_F32, "bf16": DT_BF16, "f16": DT_F16}


def build(force: bool = True) -> str:
    """Compile the oracle's C source into a shared object next to it."""
    if force or not os.path.exists(_BUILT):
        tmp = _BUILT + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _BUILT)
    return _BUILT


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) and _LIB == _BUILT:
            build()
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.orc_score.argtypes = [vp, i32, i64, i64, i32, vp, i32, vp]
        L.orc_select.argtypes = [vp, i64, i64, i64, i64, i32, vp, vp]
        L.orc_groups_update.argtypes = [i64, i64, i64, i32, i32, vp, i32, i64, i64, i64, i32,
                                        vp, vp, vp, vp, vp, vp, vp, vp, i64, vp]
        L.orc_num_threads.argtypes = []
        L.orc_set_num_threads.argtypes = [i32]
        for f in (L.orc_score, L.orc_select, L.orc_groups_update, L.orc_num_threads, L.orc_set_num_threads):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError("%s failed with code %d" % (what, rc))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dt(x: np.ndarray, dtype: Optional[str] = None) -> int:
    """Element type code of a key array: float32, or raw 16-bit bits (uint16)
    read as bf16 unless dtype says "f16"."""
    if x.dtype == np.float32:
        return DT_F32
    if x.dtype == np.uint16:
        return DT_F16 if dtype == "f16" else DT_BF16
    raise TypeError("keys must be float32 or 16-bit bits (uint16), got %s" % x.dtype)


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops over groups (timing baselines)."""
    _check(lib().orc_set_num_threads(n), "orc_set_num_threads")


def score(k: np.ndarray, mode: str = "l2", f: Optional[np.ndarray] = None, sign: int = 1,
          dtype: Optional[str] = None) -> np.ndarray:
    """Scores [n] float32 of rows k [n, D] (float32, or bf16 / f16 bits)."""
    k = np.ascontiguousarray(k)
    n, D = k.shape
    out = np.empty(n, dtype=np.float32)
    ff = None if f is None else np.ascontiguousarray(f, dtype=np.float32)
    _check(lib().orc_score(_ptr(k), _dt(k, dtype), n, D, MODE_L2 if mode == "l2" else MODE_PROJ,
                           _ptr(ff), sign, _ptr(out)), "orc_score")
    return out


def select(s: np.ndarray, budget: int, n_sink: int, recent: int, keep: str) -> np.ndarray:
    """Kept row indices (ascending, int64) of the concatenated scores s."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(max(1, s.size), dtype=np.int64)
    n_out = ctypes.c_int64(0)
    _check(lib().orc_select(_ptr(s), s.size, budget, n_sink, recent, 1 if keep == "low" else 0,
                            _ptr(out), ctypes.byref(n_out)), "orc_select")
    return out[:n_out.value].copy()


class OracleCache:
    """State of G independent groups (the kept rows of each), absorbing blocks.

    Arrays: ``k``/``v`` [G, budget, D] (float32, or uint16 bits of bf16 / f16), ``s`` [G, budget]
    float32 stored scores, ``pos`` [G, budget] int32, ``n`` [G] kept counts,
    ``tokens`` [G] tokens seen (the true offset)."""

    def __init__(self, G: int, D: int, dtype: str, budget: int, n_sink: int, recent: int,
                 keep: str, mode: str = "l2", filters: Optional[np.ndarray] = None, sign: int = 1):
        self.G, self.D, self.dtype = G, D, dtype
        self.budget, self.n_sink, self.recent, self.keep = budget, n_sink, recent, keep
        self.mode, self.sign = mode, sign
        npdt = np.float32 if dtype == "f32" else np.uint16
        self.k = np.zeros((G, budget, D), dtype=npdt)
        self.v = np.zeros((G, budget, D), dtype=npdt)
        self.s = np.zeros((G, budget), dtype=np.float32)
        self.pos = np.zeros((G, budget), dtype=np.int32)
        self.n = np.zeros(G, dtype=np.int64)
        self.tokens = np.zeros(G, dtype=np.int64)
        self.filters = None if filters is None else np.ascontiguousarray(
            np.asarray(filters, dtype=np.float32).reshape(G, D))

    def update(self, k_new: np.ndarray, v_new: np.ndarray, scores_in: Optional[np.ndarray] = None):
        k_new = np.ascontiguousarray(k_new)
        v_new = np.ascontiguousarray(v_new)
        G, S, D = k_new.shape
        assert G == self.G and D == self.D and v_new.shape == k_new.shape
        assert k_new.dtype == self.k.dtype and v_new.dtype == self.k.dtype
        if self.mode == "proj" and self.filters is None:
            raise OracleError("projection mode needs filters")
        si = None if scores_in is None else np.ascontiguousarray(scores_in, dtype=np.float32).reshape(G, S)
        _check(lib().orc_groups_update(
            G, self.budget, D, _DT[self.dtype],
            MODE_L2 if self.mode == "l2" else MODE_PROJ, _ptr(self.filters), self.sign,
            self.budget, self.n_sink, self.recent, 1 if self.keep == "low" else 0,
            _ptr(self.k), _ptr(self.v), _ptr(self.s), _ptr(self.pos), _ptr(self.n),
            _ptr(self.tokens), _ptr(k_new), _ptr(v_new), S, _ptr(si)), "orc_groups_update")

    def kept(self, g: int):
        n = int(self.n[g])
        return self.k[g, :n], self.v[g, :n], self.s[g, :n], self.pos[g, :n]

    def copy(self) -> "OracleCache":
        c = OracleCache.__new__(OracleCache)
        c.__dict__.update({k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in self.__dict__.items()})
        return c


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of float32 keys or of bf16 / fp16 bit patterns."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    bits = np.asarray(x, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class FallbackOracleCache:
    """The key-SVD fallback lifecycle of one cache of G groups (Q-Filters page,
    "How it works" step 2, "Key-SVD fallback", "Path dependence").

    * Before any filter exists nothing can be scored, so every row is held:
      the cache keeps all of its tokens, even over budget.
    * The block that brings the tokens seen to calib_tokens freezes the filter
      of each group: ``estimate_filter_dir`` (calib.py) over the held keys plus
      that block's keys (calib_keys="crossing"; different chunkings therefore
      freeze different filters), or over exactly the first calib_tokens keys
      (calib_keys="first").  The filter is stored as float32.
    * The same call then scores every held row and the block's rows with the
      frozen filter and runs the eviction step over the whole concatenation
      from an empty cache; later blocks are ordinary steps (OracleCache).

    ``filters_in`` replaces the estimate (lockstep runs), ``scores_in`` the
    scores of the crossing call's concatenation or of an ordinary block."""

    def __init__(self, G: int, D: int, dtype: str, budget: int, n_sink: int, recent: int, calib_tokens: int,
                 sign: int = 1, calib_keys: str = "crossing"):
        if calib_tokens < 2 or calib_keys not in ("crossing", "first"):
            raise OracleError("calib_tokens >= 2 and calib_keys in {crossing, first} required")
        self.G, self.D, self.dtype = G, D, dtype
        self.budget, self.n_sink, self.recent, self.sign = budget, n_sink, recent, sign
        self.calib_tokens, self.calib_keys = calib_tokens, calib_keys
        npdt = np.float32 if dtype == "f32" else np.uint16
        self.held_k = np.zeros((G, 0, D), dtype=npdt)
        self.held_v = np.zeros((G, 0, D), dtype=npdt)
        self.filters = None
        self.inner: Optional[OracleCache] = None
        self.crossing_rows = 0

    @property
    def tokens(self) -> int:
        return int(self.inner.tokens[0]) if self.inner is not None else self.held_k.shape[1]

    def update(self, k_new: np.ndarray, v_new: np.ndarray, scores_in: Optional[np.ndarray] = None,
               filters_in: Optional[np.ndarray] = None):
        if self.inner is not None:
            self.inner.update(k_new, v_new, scores_in)
            return
        k_all = np.concatenate([self.held_k, np.asarray(k_new)], axis=1)
        v_all = np.concatenate([self.held_v, np.asarray(v_new)], axis=1)
        n = k_all.shape[1]
        if n < self.calib_tokens:
            self.held_k, self.held_v = k_all, v_all
            return
        if filters_in is None:
            m = n if self.calib_keys == "crossing" else self.calib_tokens
            f = np.stack([calib.estimate_filter_dir(_widen(k_all[g, :m], self.dtype)) for g in range(self.G)])
            self.filters = f.astype(np.float32)
        else:
            self.filters = np.ascontiguousarray(np.asarray(filters_in, dtype=np.float32).reshape(self.G, self.D))
        self.crossing_rows = n
        self.inner = OracleCache(self.G, self.D, self.dtype, self.budget, self.n_sink, self.recent, "high", "proj",
                                 self.filters, self.sign)
        self.held_k = self.held_v = None
        self.inner.update(k_all, v_all, scores_in)

    def kept(self, g: int):
        """(k, v, s, pos) of group g; s is None while rows are only held."""
        if self.inner is not None:
            return self.inner.kept(g)
        n = self.held_k.shape[1]
        return self.held_k[g], self.held_v[g], None, np.arange(n, dtype=np.int32)
