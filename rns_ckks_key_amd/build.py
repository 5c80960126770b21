"""Build the gfx950 key-switching library in-tree (hipcc, one shared object).

Each source compiles to its own object under _build/ (in parallel), then one
link makes rns_ckks_key_amd/libckks_ks.so.  `build()` always recompiles every
source; `--changed-only` recompiles only sources newer than their object (or
whose headers changed), for quick rebuilds while editing host code.

Usage: python -m rns_ckks_key_amd.build [-v] [--changed-only]
(or called by __graft_entry__.build()).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libckks_ks.so")
SOURCES = ["kernels.hip", "noalloc.hip", "api.cpp"]
# the integer-throughput microbenchmark behind the vector-ALU roofline (measurement only)
RATES_LIB = os.path.join(HERE, "libckks_valu_rates.so")
RATES_SRC = "valu_rates.hip"
HEADERS = [os.path.join(CSRC, h) for h in ("ckks_internal.h", "modarith.h")] + [
    os.path.join(ROOT, "include", "ckks_ks.h")]
ARCH = os.environ.get("CKKS_OFFLOAD_ARCH", "gfx950")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 instructions are disabled for every device function (no fp32 math is used anyway)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _filtered(out: str) -> str:
    return "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip())


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = _filtered(r.stdout + r.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs:
        print(errs, flush=True)


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    return any(os.path.getmtime(f) > t for f in [src] + HEADERS)


def build(verbose: bool = False, changed_only: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    objs = []
    rates_obj = os.path.join(OBJ, RATES_SRC + ".o")
    if not changed_only or _stale(os.path.join(CSRC, RATES_SRC), rates_obj):
        jobs.append(["hipcc"] + FLAGS + ["-c", os.path.join(CSRC, RATES_SRC), "-o", rates_obj + ".tmp"])
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(OBJ, s + ".o")
        objs.append(obj)
        if not changed_only or _stale(src, obj):
            # hipcc compiles every source as HIP (host and gfx950 passes)
            jobs.append(["hipcc"] + FLAGS + ["-c", src, "-o", obj + ".tmp"])
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    for c in jobs:
        os.replace(c[-1], c[-1][:-4])
    tmp = LIB + ".tmp"
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    _run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", RATES_LIB + ".tmp", rates_obj], verbose)
    os.replace(RATES_LIB + ".tmp", RATES_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, changed_only="--changed-only" in sys.argv))
