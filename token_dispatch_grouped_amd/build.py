"""Build libmoe.so and libmoe_debug.so (all HIP sources, gfx950) in the package directory.

Every source is compiled to its own object in parallel, then linked. The debug
library is the same objects except for the sources that test MOE_DEBUG, which
are compiled a second time with it defined: in that build the dispatch also
writes a device error word for out-of-range expert ids (see include/moe.h).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe.so")
LIB_DEBUG = os.path.join(PKG, "libmoe_debug.so")
OBJ_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# the host pass does not know the packed-fp32 feature and says so; that is harmless
_NOISE = "is not a recognized feature for this target"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def _uses_debug(src: str) -> bool:
    with open(src) as f:
        return "MOE_DEBUG" in f.read()


def _run(cmd: list[str]) -> str:
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if _NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    return err


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link both libraries; returns the
    release library's path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    jobs = []  # (source, object, extra flags)
    for s in srcs:
        stem = os.path.splitext(os.path.basename(s))[0]
        jobs.append((s, os.path.join(OBJ_DIR, stem + ".o"), []))
        if _uses_debug(s):
            jobs.append((s, os.path.join(OBJ_DIR, stem + ".debug.o"), ["-DMOE_DEBUG=1"]))

    def compile_one(job):
        src, obj, extra = job
        cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return _run(cmd)

    # the slowest sources first, so the pool does not end on one long compile
    jobs.sort(key=lambda j: -os.path.getsize(j[0]))
    with ThreadPoolExecutor(_jobs()) as ex:
        for err in ex.map(compile_one, jobs):
            if err.strip() and verbose:
                print(err, file=sys.stderr)
    release = [o for _, o, extra in jobs if not extra]
    debug_of = {s: o for s, o, extra in jobs if extra}
    debug = [debug_of.get(s, o) for s, o, extra in jobs if not extra]
    for lib, objs in ((LIB, release), (LIB_DEBUG, debug)):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *sorted(objs)]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
