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


if __name__ == "__main__":
    print(build(verbose=True))
