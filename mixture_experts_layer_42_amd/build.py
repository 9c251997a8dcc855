"""Build the HIP library ``libmoe.so`` in-tree for gfx950.

    python -m mixture_experts_layer_42_amd.build

Every HIP translation unit is compiled with packed-FP32 instructions disabled, and the
routing unit additionally with floating-point contraction off (its routing score is a
fixed sequence of separately rounded float32 operations).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
PEAK_LIB = os.path.join(PKG, "libmoe_peak.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

UNITS = {
    "route.hip": ["-ffp-contract=off"],
    "gemm.hip": [],
    "move.hip": [],
    "moe_api.cpp": [],
    "debug.hip": [],
}
PEAK_UNITS = {"peak.hip": []}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libmoe.so)")


def common_flags():
    return ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


def _compile(unit, extra, verbose):
    src = os.path.join(CSRC, unit)
    obj = os.path.join(BUILD, unit + ".o")
    cmd = [hipcc()] + common_flags() + extra + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {unit} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build_library(verbose: bool = False) -> str:
    """Compile every unit and link libmoe.so (the layer) and libmoe_peak.so (the
    achievable-peak microbenchmarks the bench reports) next to this file. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    units = dict(UNITS)
    units.update(PEAK_UNITS)
    with ThreadPoolExecutor(max_workers=len(units)) as ex:
        objs = dict(zip(units, ex.map(lambda kv: _compile(kv[0], kv[1], verbose), units.items())))
    _link([objs[u] for u in UNITS], LIB, verbose)
    _link([objs[u] for u in PEAK_UNITS], PEAK_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
