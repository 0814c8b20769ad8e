"""Builds libmot.so (HIP, gfx950) in-tree with hipcc.

Flags: -O3, no fast math, -ffp-contract=off (no FMA contraction outside the
MFMA), correctly rounded fp32 divide and sqrt (hipcc's default, kept), and
packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmot.so")
SOURCES = [os.path.join(CSRC, "mot_kernels.hip"), os.path.join(CSRC, "mot_attention.hip"),
           os.path.join(CSRC, "mot_latent.hip"), os.path.join(CSRC, "mot_api.cpp")]
HEADERS = [os.path.join(CSRC, "mot_internal.h"),
           os.path.join(os.path.dirname(HERE), "include", "mot.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Werror=return-type",
]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libmot.so; returns its path.  Always recompiles when force."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    _write_build_info()
    return LIB


def _write_build_info():
    """Record the source revision the library was built from (the GPU run
    has no git history)."""
    import json
    root = os.path.dirname(HERE)
    try:
        rev = subprocess.run(["git", "rev-parse", "--short", "HEAD"], cwd=root, capture_output=True,
                             text=True).stdout.strip() or "unknown"
        dirty = subprocess.run(["git", "status", "--porcelain", "--", "mixture_transformers_token_amd",
                                "include"], cwd=root, capture_output=True, text=True).stdout.strip() != ""
    except Exception:
        rev, dirty = "unknown", None
    with open(os.path.join(HERE, "BUILD_INFO.json"), "w") as f:
        json.dump({"commit": rev, "dirty": dirty}, f)


if __name__ == "__main__":
    print(build(force=True, verbose=True))
