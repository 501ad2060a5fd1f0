"""Build step: compiles the HIP sources under csrc/ into the in-tree shared library
libgptq_mi355x.so for gfx950 (hipcc cross-compiles, no GPU needed)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgptq_mi355x.so")
SOURCES = ["api.cpp", "repack.hip", "skinny.hip", "tiled.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-result",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into LIB (always rebuilds).  Returns the library path."""
    tmp = LIB + ".tmp"
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        # api.cpp holds host code only but calls the HIP runtime: compile it as HIP too
        srcs += (["-x", "hip", p] if s.endswith(".hip") or s.endswith(".cpp") else [p])
    cmd = [HIPCC] + hipcc_flags() + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
