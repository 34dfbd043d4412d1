"""ctypes loader for libkvevict.so (the C ABI declared in include/kvevict.h).

torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process: device pointers and streams are then
interchangeable).  A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvevict.so")

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

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "kvx_last_error": ([], ctypes.c_char_p),
    "kvx_abi_version": ([], ctypes.c_int),
    "qf_score_keys": ([_vp, KvxShape, _i64, _i32, _vp, _i32, _vp, _vp], ctypes.c_int),
    "kv_evict_workspace_size": ([KvxShape, _i64, _i64, KvxParams, ctypes.POINTER(_sz)], ctypes.c_int),
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
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        try:
            import torch  # noqa: F401  (binds the library to torch's HIP runtime)
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkvevict.so is not built (expected at %s); run "
                              "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def check(fn: str, rc: int) -> None:
    if rc != KVX_OK:
        raise KvxError(fn, rc, lib().kvx_last_error().decode(errors="replace"))


def call(fn: str, *args) -> None:
    check(fn, getattr(lib(), fn)(*args))
