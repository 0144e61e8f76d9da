"""Build libffnq.so (gfx950) in-tree with hipcc.

Usage: python -m moe_expert_dequant_amd.build   (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libffnq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "ffnq.hip")]
HEADERS = [os.path.join(CSRC, h) for h in ("device.h", "prefill.h", "qgemm.h", "route.h", "stream.h", "tail.h", "tiled.h")] + [
    os.path.join(ROOT, "include", "ffnq.h")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    # packed fp32 VALU ops stay off: the compiler may not form them from scalar or float2 code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libffnq.so; returns its path.  Always recompiles when force."""
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in SOURCES + HEADERS)
        if os.path.getmtime(LIB) >= newest:
            return LIB
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
