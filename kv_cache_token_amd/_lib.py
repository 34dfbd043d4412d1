"""ctypes loader for libkvevict.so (the C ABI declared in include/kvevict.h).

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process: device pointers and streams are then
interchangeable).  A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# KVX_LIB names another build of the same library (the host-sanitizer build
# under _build/asan/); by default the in-tree libkvevict.so.
LIB_PATH = os.environ.get("KVX_LIB") or os.path.join(HERE, "libkvevict.so")
CHECK_LIB_PATH = os.path.join(HERE, "libkvevict_check.so")   # built with -DKVX_CHECK

KVX_OK, KVX_EINVAL, KVX_ERANGE, KVX_EDEVICE, KVX_EIO, KVX_EMISMATCH = 0, -1, -2, -3, -4, -5
KVX_F32, KVX_BF16, KVX_F16 = 0, 1, 2
KVX_SCORE_L2, KVX_SCORE_PROJ, KVX_SCORE_CACHE_KEYS = 0, 1, 0x100
KVX_KEEP_HIGH, KVX_KEEP_LOW = 0, 1
KVX_HEAD_DIM, KVX_MAX_BUDGET, KVX_MAX_TOTAL, KVX_ONCHIP_TOTAL = 128, 1 << 21, 1 << 22, 1 << 18
KVX_NOALLOC_SCRATCH_BYTES = 8 << 20

_CODES = {KVX_EINVAL: "EINVAL", KVX_ERANGE: "ERANGE", KVX_EDEVICE: "EDEVICE", KVX_EIO: "EIO",
          KVX_EMISMATCH: "EMISMATCH"}


class KvxShape(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("B", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class KvxParams(ctypes.Structure):
    _fields_ = [("budget", ctypes.c_int64), ("n_sink", ctypes.c_int64), ("recent", ctypes.c_int64),
                ("keep", ctypes.c_int32)]


class KvxStats(ctypes.Structure):
    _fields_ = [("kept_bytes", ctypes.c_int64), ("full_seq_bytes", ctypes.c_int64),
                ("compression_ratio", ctypes.c_double), ("tokens_seen", ctypes.c_int64),
                ("tokens_kept", ctypes.c_int64), ("filter_bytes", ctypes.c_int64)]


class KvxError(RuntimeError):
    """A libkvevict call returned an error status."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s failed (%s): %s" % (fn, _CODES.get(code, code), msg))
        self.code = code


_lib = None
_loaded = {}      # path -> CDLL
_use_checked = False

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "kvx_last_error": ([], ctypes.c_char_p),
    "kvx_abi_version": ([], ctypes.c_int),
    "qf_score_keys": ([_vp, KvxShape, _i64, _i32, _vp, _i32, _vp, _vp], ctypes.c_int),
    "kv_evict_workspace_size": ([KvxShape, _i64, _i64, KvxParams, ctypes.POINTER(_sz)], ctypes.c_int),
    "kv_score_append": ([_vp, _vp, KvxShape, _i64, _i32, _vp, _i32, _i64, _i64, KvxParams, _vp, _vp, _vp, _vp,
                         _vp, _vp], ctypes.c_int),
    "kv_evict_topk": ([_vp, _vp, KvxShape, _i64, _i64, KvxParams, _vp, _vp, _sz, _vp], ctypes.c_int),
    "kv_evict_topk_noalloc": ([_vp, _vp, KvxShape, _i64, _i64, KvxParams, _vp, _vp], ctypes.c_int),
    "kv_compact_gather": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, KvxShape, _i64, _i64, KvxParams,
                           _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "kv_evict_one_inplace": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, KvxShape, _i64, KvxParams, _vp],
                             ctypes.c_int),
    "qf_filters_load": ([ctypes.c_char_p, ctypes.c_char_p, _i64, _i64, _i64, _vp, ctypes.POINTER(_i64)],
                        ctypes.c_int),
    "qf_filters_save": ([ctypes.c_char_p, _vp, _i64, _i64, _i64, ctypes.c_char_p, _i64, ctypes.c_char_p],
                        ctypes.c_int),
    "qf_filters_from_queries": ([_vp, _i64, _i64, _i64, _i64, _vp], ctypes.c_int),
    "qf_filters_from_keys": ([_vp, _i32, _i64, _i64, _i64, _i64, _vp], ctypes.c_int),
    "kv_passthrough_append": ([_vp, _vp, _i64, _i64, _vp, _vp, _i64, KvxShape, _vp, _vp, _vp, _i64, _vp],
                              ctypes.c_int),
    "qf_filters_from_keys_device": ([_vp, _i32, _i64, _i64, _i64, _i64, _vp, _vp, _i32, _vp], ctypes.c_int),
    "qf_filters_from_queries_device": ([_vp, _i32, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _i32, _vp],
                                       ctypes.c_int),
    "kvx_stats": ([KvxShape, _i64, _i64, _i32, ctypes.POINTER(KvxStats)], ctypes.c_int),
    "kvx_check_status_word": ([_vp], ctypes.c_int),
}
KVX_CHECK_SLOT, KVX_CHECK_RANGE, KVX_CHECK_ORDER, KVX_CHECK_COUNT = 1, 2, 3, 4


def _load(path: str):
    if path not in _loaded:
        try:
            import torch  # noqa: F401  (binds the library to torch's HIP runtime)
        except ImportError:
            pass
        if not os.path.exists(path):
            raise ImportError("%s is not built (expected at %s); run "
                              "`python -c 'import __graft_entry__ as g; g.build()'`" % (os.path.basename(path), path))
        L = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _loaded[path] = L
    return _loaded[path]


def lib():
    """The library every binding call goes to (raises if it has not been
    built): libkvevict.so, or its checked build inside ``checked()``."""
    global _lib
    if _use_checked:
        return _load(CHECK_LIB_PATH)
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


class checked:
    """Context manager: calls made (or prepared) inside go to the checked build
    (libkvevict_check.so, -DKVX_CHECK), which records index-list violations in
    the status words given to kvx_check_status_word."""

    def __enter__(self):
        global _use_checked
        self._prev = _use_checked
        _load(CHECK_LIB_PATH)
        _use_checked = True
        return _load(CHECK_LIB_PATH)

    def __exit__(self, *exc):
        global _use_checked
        _use_checked = self._prev
        return False


def check(fn: str, rc: int) -> None:
    if rc != KVX_OK:
        raise KvxError(fn, rc, lib().kvx_last_error().decode(errors="replace"))


def call(fn: str, *args) -> None:
    check(fn, getattr(lib(), fn)(*args))
