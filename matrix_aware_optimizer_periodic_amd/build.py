"""Compile the gfx950 HIP library in-tree: ``libmuon_hip.so`` next to this file.

Usage: ``python -m matrix_aware_optimizer_periodic_amd.build`` (or call
``build()``).  Objects go to ``_build/``; every call recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libmuon_hip.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["kernels_rownorm.hip", "kernels_ns5.hip", "kernels_gram_tri.hip", "kernels_misc.hip",
           "noalloc.hip", "runtime.cpp"]
ARCH = os.environ.get("MUON_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include"]
# Keep hipcc from forming packed fp32 arithmetic in device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [HIPCC, *DEVICE, *COMMON, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, "-x", "c++", *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    # A kernel whose launch stub the host pass dropped still links (the
    # library is shared) and only fails when loaded: refuse it here.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "muon" in ln]
    if missing:
        os.remove(tmp)
        raise RuntimeError(f"library has undefined symbols of its own: {missing[:4]}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
