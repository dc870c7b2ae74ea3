"""Build the KDA HIP library (gfx950) in-tree: kda_gated_delta_core_amd/libkda_amd.so."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda_amd.so")
SOURCES = ["kda_api.cpp", "kda_recurrent.hip", "kda_chunk.hip", "kda_norm.hip", "kda_front_end.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed FP32 instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _link(lib: str, sources: list, verbose: bool) -> None:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for s in sources:
        o = os.path.join(objdir, os.path.basename(s) + ".o")
        cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip", "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd))
        subprocess.run(cmd, check=True)
        objs.append(o)
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, lib)


def build(force: bool = True, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    deps = srcs + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps.append(os.path.join(ROOT, "include", "kda.h"))
    stale = lambda lib, d: not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(x) for x in d)
    if force or stale(LIB, deps):
        _link(LIB, srcs, verbose)
    return LIB


if __name__ == "__main__":
    print(build(force="--if-stale" not in sys.argv, verbose="-v" in sys.argv))
