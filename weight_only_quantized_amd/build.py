"""Build step: compiles the HIP sources under csrc/ into the in-tree shared library
libgptq_mi355x.so for gfx950 (hipcc cross-compiles, no GPU needed)."""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgptq_mi355x.so")
SOURCES = ["api.cpp", "repack.hip", "skinny.hip", "skinny_b2.hip", "skinny_b3.hip", "skinny_b4.hip",
           "skinny_b5.hip", "skinny_b6.hip", "skinny_b7.hip", "skinny_b8.hip", "mid.hip", "mid_b2.hip", "mid_b3.hip",
           "mid_b4.hip", "mid_b5.hip", "mid_b6.hip", "mid_b7.hip", "mid_b8.hip", "tiled.hip", "quantize.hip",
           "read_floor.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-result",
    ]


def spilled_kernels(remarks: str) -> list:
    """Kernels whose resource-usage remarks report VGPR or SGPR spills.  Every kernel here is
    sized to stay in registers; a spill means a configuration outgrew its budget."""
    out, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"[SV]GPRs Spill: (\d+)", line)
        if m and int(m.group(1)) > 0 and name and name not in out:
            out.append(name)
    return out


def undefined_kernel_stubs(lib: str) -> list:
    """Kernel launch stubs the library references but does not define.  hipcc's host pass can drop
    a kernel's stub without a diagnostic (seen with some buffer-to-LDS builtin arguments); the
    library then fails to load, so the build checks for it instead."""
    try:
        r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    except FileNotFoundError:
        return []
    return [ln.split()[-1] for ln in r.stdout.splitlines() if "__device_stub__" in ln]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel, one hipcc per file) and link LIB.  Always rebuilds.
    Returns the library path."""
    import concurrent.futures
    import tempfile
    jobs = jobs or min(8, os.cpu_count() or 1)
    objdir = tempfile.mkdtemp(prefix="gq_build_")
    flags = [f for f in hipcc_flags() if f != "-shared"]

    def compile_one(s):
        src = os.path.join(CSRC, s)
        obj = os.path.join(objdir, s + ".o")
        # api.cpp holds host code only but calls the HIP runtime: compile it as HIP too
        cmd = [HIPCC] + flags + ["-x", "hip", "-c", src, "-o", obj, "-Rpass-analysis=kernel-resource-usage"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {s} ({r.returncode})")
        spills = spilled_kernels(r.stderr)
        if spills:
            raise RuntimeError(f"{s}: kernels spill registers to scratch (not allowed): {spills}")
        return obj

    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"link failed ({r.returncode})")
    missing = undefined_kernel_stubs(tmp)
    if missing:
        os.remove(tmp)
        raise RuntimeError(f"kernels without a host launch stub (the host pass dropped them): {missing[:4]}")
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    os.rmdir(objdir)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
