"""Python binding of libkvevict with the C ABI's names (argument marshalling only).

Device entry points take torch CUDA tensors (torch is used for device memory and
streams only; every step of the eviction path runs in the library's HIP
kernels).  Shapes and element types are checked here before a pointer is
handed to the library, because a kernel cannot check the size of a buffer.
Host entry points take and return numpy arrays.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib
from ._lib import (KVX_BF16, KVX_F16, KVX_F32, KVX_HEAD_DIM, KVX_KEEP_HIGH, KVX_KEEP_LOW, KVX_SCORE_CACHE_KEYS,
                   KVX_SCORE_L2, KVX_SCORE_PROJ, KvxParams, KvxShape, KvxStats, call)

D = KVX_HEAD_DIM


def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    if dtype in ("bf16", torch.bfloat16, KVX_BF16):
        return KVX_BF16
    if dtype in ("f16", torch.float16, KVX_F16):
        return KVX_F16
    if dtype in ("f32", torch.float32, KVX_F32):
        return KVX_F32
    raise ValueError("unsupported K/V dtype %r (bf16, f16 or f32)" % (dtype,))


def torch_dtype(code: int):
    torch = _torch()
    return {KVX_BF16: torch.bfloat16, KVX_F16: torch.float16, KVX_F32: torch.float32}[code]


def make_shape(L: int, B: int, H: int, dtype, D_: int = D) -> KvxShape:
    return KvxShape(L, B, H, D_, dtype_code(dtype))


def make_params(budget: int, n_sink: int, recent: int, keep) -> KvxParams:
    k = {"high": KVX_KEEP_HIGH, "low": KVX_KEEP_LOW}.get(keep, keep)
    return KvxParams(budget, n_sink, recent, k)


def mode_code(mode) -> int:
    return {"l2": KVX_SCORE_L2, "proj": KVX_SCORE_PROJ}.get(mode, mode)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dev(t, name: str, dtype, numel: int, allow_none: bool = False):
    """Pointer of a contiguous CUDA tensor with the expected element type and at
    least `numel` elements (None allowed only when the library does not read it)."""
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < numel:
        raise ValueError("%s holds %d elements, needs %d" % (name, t.numel(), numel))
    return t.data_ptr() if numel > 0 else (t.data_ptr() or None)


def _G(shape: KvxShape) -> int:
    return shape.L * shape.B * shape.H


def _dispatch(fn: str, args, prepare: bool):
    """Call the library now, or (prepare=True) return (function, args) so that a
    validated call can be replayed later without re-marshalling."""
    if prepare:
        return getattr(_lib.lib(), fn), tuple(args)
    call(fn, *args)
    return None


def run_prepared(calls) -> None:
    """Replay prepared calls in order (each was validated when prepared)."""
    for f, args in calls:
        rc = f(*args)
        if rc != 0:
            _lib.check(f.__name__, rc)


# --------------------------------------------------------------------------- device


def qf_score_keys(k_new, shape: KvxShape, S: int, mode, filters, sign: int, s_new, stream=None,
                  prepare: bool = False, cache_keys: bool = False):
    """Score G*S incoming rows into s_new [G, S] (float32); cache_keys reads the
    keys with cache-allocating loads (KVX_SCORE_CACHE_KEYS)."""
    torch = _torch()
    G, m = _G(shape), mode_code(mode)
    kp = _dev(k_new, "k_new", torch_dtype(shape.dtype), G * S * shape.D)
    fp = _dev(filters, "filters", torch.float32, shape.L * shape.H * shape.D, allow_none=(m == KVX_SCORE_L2))
    sp = _dev(s_new, "s_new", torch.float32, G * S)
    mf = m | KVX_SCORE_CACHE_KEYS if cache_keys else m
    return _dispatch("qf_score_keys", (kp, shape, S, mf, fp, sign, sp, _stream(stream)), prepare)


def kv_score_append(k_new, v_new, shape: KvxShape, S: int, mode, filters, sign: int, pos_base: int, n_kept: int,
                    params: KvxParams, k_cache, v_cache, s_cache, pos_cache, s_new=None, stream=None,
                    prepare: bool = False):
    """Score the S incoming rows and append them after the n_kept kept rows in
    one pass (a call that evicts nothing: n_kept + S <= budget)."""
    torch = _torch()
    G, m, td, cap, Dd = _G(shape), mode_code(mode), torch_dtype(shape.dtype), params.budget, shape.D
    args = (_dev(k_new, "k_new", td, G * S * Dd), _dev(v_new, "v_new", td, G * S * Dd), shape, S, m,
            _dev(filters, "filters", torch.float32, shape.L * shape.H * Dd, allow_none=(m == KVX_SCORE_L2)), sign,
            pos_base, n_kept, params,
            _dev(k_cache, "k_cache", td, G * cap * Dd), _dev(v_cache, "v_cache", td, G * cap * Dd),
            _dev(s_cache, "s_cache", torch.float32, G * cap), _dev(pos_cache, "pos_cache", torch.int32, G * cap),
            _dev(s_new, "s_new", torch.float32, G * S, allow_none=True), _stream(stream))
    return _dispatch("kv_score_append", args, prepare)


def kv_evict_workspace_size(shape: KvxShape, n_kept: int, S: int, params: KvxParams) -> int:
    n = ctypes.c_size_t(0)
    call("kv_evict_workspace_size", shape, n_kept, S, params, ctypes.byref(n))
    return n.value


def kv_evict_topk(s_kept, s_new, shape: KvxShape, n_kept: int, S: int, params: KvxParams, keep_idx,
                  ws=None, stream=None, prepare: bool = False):
    torch = _torch()
    G = _G(shape)
    kp = _dev(s_kept, "s_kept", torch.float32, G * params.budget, allow_none=(n_kept == 0))
    np_ = _dev(s_new, "s_new", torch.float32, G * S, allow_none=(S == 0))
    ip = _dev(keep_idx, "keep_idx", torch.int32, G * params.budget)
    wp = _dev(ws, "ws", torch.uint8, 0, allow_none=True)  # its size is checked by the library
    wsb = 0 if ws is None else ws.numel()
    return _dispatch("kv_evict_topk", (kp, np_, shape, n_kept, S, params, ip, wp, wsb, _stream(stream)), prepare)


def kv_evict_topk_noalloc(s_kept, s_new, shape: KvxShape, n_kept: int, S: int, params: KvxParams, keep_idx,
                          stream=None, prepare: bool = False):
    """kv_evict_topk without a workspace argument: the library's static device
    scratch serves the selections that need one (allocation-free callers)."""
    torch = _torch()
    G = _G(shape)
    kp = _dev(s_kept, "s_kept", torch.float32, G * params.budget, allow_none=(n_kept == 0))
    np_ = _dev(s_new, "s_new", torch.float32, G * S, allow_none=(S == 0))
    ip = _dev(keep_idx, "keep_idx", torch.int32, G * params.budget)
    return _dispatch("kv_evict_topk_noalloc", (kp, np_, shape, n_kept, S, params, ip, _stream(stream)), prepare)


def kv_compact_gather(k_kept, v_kept, s_kept, pos_kept, k_new, v_new, s_new, pos_base: int, keep_idx,
                      shape: KvxShape, n_kept: int, S: int, params: KvxParams, k_out, v_out, s_out, pos_out,
                      stream=None, prepare: bool = False):
    torch = _torch()
    G, td, cap, Dd = _G(shape), torch_dtype(shape.dtype), params.budget, shape.D
    evict = n_kept + S > cap
    args = [
        _dev(k_kept, "k_kept", td, G * cap * Dd, allow_none=(n_kept == 0)),
        _dev(v_kept, "v_kept", td, G * cap * Dd, allow_none=(n_kept == 0)),
        _dev(s_kept, "s_kept", torch.float32, G * cap, allow_none=(n_kept == 0)),
        _dev(pos_kept, "pos_kept", torch.int32, G * cap, allow_none=(n_kept == 0)),
        _dev(k_new, "k_new", td, G * S * Dd, allow_none=(S == 0)),
        _dev(v_new, "v_new", td, G * S * Dd, allow_none=(S == 0)),
        _dev(s_new, "s_new", torch.float32, G * S, allow_none=(S == 0)),
        pos_base,
        _dev(keep_idx, "keep_idx", torch.int32, G * cap, allow_none=not evict),
        shape, n_kept, S, params,
        _dev(k_out, "k_out", td, G * cap * Dd),
        _dev(v_out, "v_out", td, G * cap * Dd),
        _dev(s_out, "s_out", torch.float32, G * cap),
        _dev(pos_out, "pos_out", torch.int32, G * cap),
        _stream(stream),
    ]
    return _dispatch("kv_compact_gather", args, prepare)


def kv_evict_one_inplace(k_cache, v_cache, s_cache, pos_cache, k_new, v_new, s_new, pos_base: int,
                         shape: KvxShape, n_kept: int, params: KvxParams, stream=None, prepare: bool = False):
    torch = _torch()
    G, td, cap, Dd = _G(shape), torch_dtype(shape.dtype), params.budget, shape.D
    args = (_dev(k_cache, "k_cache", td, G * cap * Dd), _dev(v_cache, "v_cache", td, G * cap * Dd),
            _dev(s_cache, "s_cache", torch.float32, G * cap), _dev(pos_cache, "pos_cache", torch.int32, G * cap),
            _dev(k_new, "k_new", td, G * Dd), _dev(v_new, "v_new", td, G * Dd),
            _dev(s_new, "s_new", torch.float32, G), pos_base, shape, n_kept, params, _stream(stream))
    return _dispatch("kv_evict_one_inplace", args, prepare)


def kv_passthrough_append(k_held, v_held, n_held: int, cap_held: int, k_new, v_new, S: int, shape: KvxShape,
                          k_out, v_out, pos_out, cap_out: int, stream=None, prepare: bool = False):
    """Pre-calibration passthrough: held rows then new rows into the output
    (in place when the output is the held buffer)."""
    torch = _torch()
    G, td, Dd = _G(shape), torch_dtype(shape.dtype), shape.D
    args = (_dev(k_held, "k_held", td, G * cap_held * Dd, allow_none=(n_held == 0)),
            _dev(v_held, "v_held", td, G * cap_held * Dd, allow_none=(n_held == 0)), n_held, cap_held,
            _dev(k_new, "k_new", td, G * S * Dd, allow_none=(S == 0)),
            _dev(v_new, "v_new", td, G * S * Dd, allow_none=(S == 0)), S, shape,
            _dev(k_out, "k_out", td, G * cap_out * Dd), _dev(v_out, "v_out", td, G * cap_out * Dd),
            _dev(pos_out, "pos_out", torch.int32, G * cap_out), cap_out, _stream(stream))
    return _dispatch("kv_passthrough_append", args, prepare)


def qf_filters_from_keys_device(k, G: int, n: int, group_stride: int, out, status, max_iter: int = 20000,
                                stream=None, prepare: bool = False):
    """Key-SVD fallback filters of G groups on the device: out [G, D] float32,
    status [G] int32 (0 converged, 1 not separated within max_iter, 2 zero)."""
    torch = _torch()
    code = dtype_code(k.dtype)
    Dd = k.shape[-1]
    args = (_dev(k, "k", torch_dtype(code), (G - 1) * group_stride * Dd + n * Dd if G else 0), code, G, n,
            group_stride, Dd, _dev(out, "out", torch.float32, G * Dd), _dev(status, "status", torch.int32, G),
            max_iter, _stream(stream))
    return _dispatch("qf_filters_from_keys_device", args, prepare)


def qf_filters_from_queries_device(q, H_kv: int, out, status, max_iter: int = 20000, stream=None,
                                   prepare: bool = False):
    """Query-SVD calibration on the device: q [L, H_q, N, D] activations ->
    out [L, H_kv, D] float32 filters, status [L, H_kv] int32."""
    torch = _torch()
    code = dtype_code(q.dtype)
    L, Hq, N, Dd = q.shape
    args = (_dev(q, "q", torch_dtype(code), L * Hq * N * Dd), code, L, Hq, N, Dd, H_kv,
            _dev(out, "out", torch.float32, L * H_kv * Dd), _dev(status, "status", torch.int32, L * H_kv),
            max_iter, _stream(stream))
    return _dispatch("qf_filters_from_queries_device", args, prepare)


def kvx_check_status_word(status) -> None:
    """Checked build only: record index-list violations in `status` (a CUDA
    int32 tensor of 4 words the caller zeroes; None stops the recording)."""
    torch = _torch()
    call("kvx_check_status_word", _dev(status, "status", torch.int32, 4, allow_none=True))


# --------------------------------------------------------------------------- host


def qf_filters_load(path: str, L: int, H_kv: int, expect_model_id: Optional[str] = None,
                    D_: int = D) -> Tuple[np.ndarray, int]:
    out = np.empty((L, H_kv, D_), dtype=np.float32)
    ns = ctypes.c_int64(0)
    call("qf_filters_load", path.encode(), None if expect_model_id is None else expect_model_id.encode(),
         L, H_kv, D_, out.ctypes.data, ctypes.byref(ns))
    return out, ns.value


def qf_filters_save(path: str, filters: np.ndarray, model_id: str, n_samples: int, dataset: str) -> None:
    f = np.ascontiguousarray(filters, dtype=np.float32)
    L, H, Dd = f.shape
    call("qf_filters_save", path.encode(), f.ctypes.data, L, H, Dd, model_id.encode(), n_samples,
         dataset.encode())


def qf_filters_from_queries(q: np.ndarray, H_kv: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.float32)
    Hq, N, Dd = q.shape
    out = np.empty((H_kv, Dd), dtype=np.float32)
    call("qf_filters_from_queries", q.ctypes.data, Hq, N, Dd, H_kv, out.ctypes.data)
    return out


def qf_filters_from_keys(k: np.ndarray, n: int, dtype: str = "bf16") -> np.ndarray:
    """k: [G, rows, D] float32, or uint16 bits of bf16 / f16 (per `dtype`); uses
    each group's first n rows."""
    k = np.ascontiguousarray(k)
    G, rows, Dd = k.shape
    if k.dtype not in (np.float32, np.uint16):
        raise TypeError("keys must be float32 or 16-bit bits (uint16)")
    if k.dtype == np.uint16 and dtype not in ("bf16", "f16"):
        raise ValueError("16-bit key bits need dtype 'bf16' or 'f16', got %r" % (dtype,))
    dt = KVX_F32 if k.dtype == np.float32 else (KVX_F16 if dtype == "f16" else KVX_BF16)
    out = np.empty((G, Dd), dtype=np.float32)
    call("qf_filters_from_keys", k.ctypes.data, dt, G, n, rows, Dd, out.ctypes.data)
    return out


def kvx_stats(shape: KvxShape, tokens_seen: int, tokens_kept: int, mode) -> dict:
    st = KvxStats()
    call("kvx_stats", shape, tokens_seen, tokens_kept, mode_code(mode), ctypes.byref(st))
    return {f: getattr(st, f) for f, _ in KvxStats._fields_}


def exported_names() -> Sequence[str]:
    return list(_lib._SIGS)
