"""Build libkvevict.so (HIP kernels for gfx950 + host code) in the package directory."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvevict.so")
# The checked build (-DKVX_CHECK): the same sources, verifying the index lists
# the selection writes and the compaction reads (kvx_check_status_word).
LIB_CHECK = os.path.join(HERE, "libkvevict_check.so")
OBJ_CHECK = os.path.join(ROOT, "_build", "check")
SOURCES = ["kvx_device.hip", "kvx_calib.hip", "kvx_host.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, defines=(), out: str = LIB, objdir: str = CSRC) -> str:
    """Compile every source and link the shared library; returns its path.
    `defines` are extra -D flags (the kernels' compile-time tuning knobs)."""
    objs = []
    dflags = ["-D" + d for d in defines]
    os.makedirs(objdir, exist_ok=True)
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(objdir, src + ".o")
        if src.endswith(".hip"):
            cmd = [HIPCC, *DEVICE_FLAGS, *COMMON, *dflags, "-c", path, "-o", obj]
        else:
            cmd = ["g++", *COMMON, "-Wall", "-Wextra", "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *DEVICE_FLAGS, "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


# Host-side sanitizer build (CPU only: AddressSanitizer and UndefinedBehavior-
# Sanitizer on the library's host code and on the oracle, with clang's shared
# sanitizer runtime).  The HIP files' device code is built as usual (GPU code
# is not sanitized); each sanitizer flag on a hipcc line applies to the host
# pass alone.
SAN_DIR = os.path.join(ROOT, "_build", "asan")
LLVM_BIN = os.environ.get("KVX_LLVM_BIN", "/opt/rocm/llvm/bin")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def sanitizer_runtime() -> str:
    """Path of clang's shared ASan runtime (it carries the UBSan handlers too)."""
    out = subprocess.check_output([os.path.join(LLVM_BIN, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"])
    return out.decode().strip()


def build_sanitized(verbose: bool = False) -> dict:
    """_build/asan/libkvevict.so and _build/asan/libkvx_oracle.so; returns the
    environment that makes the tests load them (see README)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(SAN_DIR, src + ".o")
        extra = [] if src.endswith(".hip") else ["-x", "c++"]
        cmd = [HIPCC, *DEVICE_FLAGS, *COMMON, *SAN_HOST, *extra, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.check_call(cmd)
        objs.append(obj)
    lib = os.path.join(SAN_DIR, "libkvevict.so")
    san_link = ["-fsanitize=address,undefined", "-shared-libsan"]
    cmd = [os.path.join(LLVM_BIN, "clang++"), "-shared", "-fPIC", *objs, "-o", lib, *san_link,
           "-L/opt/rocm/lib", "-lamdhip64", "-lpthread", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    orc = os.path.join(SAN_DIR, "libkvx_oracle.so")
    cmd = [os.path.join(LLVM_BIN, "clang"), "-O1", "-g", "-std=c11", "-fPIC", "-shared", *san_link,
           os.path.join(ROOT, "oracle", "kvx_oracle.c"), "-o", orc, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.check_call(cmd)
    return {"LD_PRELOAD": sanitizer_runtime(), "ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0",
            "KVX_LIB": lib, "KVX_ORACLE_LIB": orc}


def build_all(verbose: bool = False) -> None:
    """The library and its checked build."""
    build(verbose)
    build(verbose, defines=("KVX_CHECK",), out=LIB_CHECK, objdir=OBJ_CHECK)


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        env = build_sanitized(verbose=True)
        print(" ".join("%s=%s" % kv for kv in env.items()))
    else:
        build_all(verbose=True)
