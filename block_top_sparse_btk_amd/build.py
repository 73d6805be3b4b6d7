"""Build libbtk.so (HIP kernels + C ABI) for gfx950, in-tree, with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "centroid.hip", "select.hip", "attend.hip", "step.hip", "token.hip",
           "probe.hip", "sketch.hip"]
LIB = os.path.join(HERE, "libbtk.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE,
    "-Wno-unused-parameter",
    # hipcc -O3 forms packed fp32 instructions from scalar float code by itself;
    # keep them out of every kernel.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False, extra=()) -> str:
    objs = []
    for src in SOURCES:
        obj = os.path.join(HERE, "_build", src.replace(".hip", ".o"))
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
