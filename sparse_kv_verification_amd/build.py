"""Build libdustin.so (the gfx950 sparse-verification library) in-tree.

hipcc compiles each HIP source for gfx950 and links one shared library next
to this file; no GPU is needed to build.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdustin.so")
SOURCES = ["attn.hip", "score.hip", "select.hip", "eval.hip", "window.hip", "pages.hip", "search.hip", "probe.hip",
           "api.hip"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, verbose, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


TRACE_LIB = os.path.join(HERE, "libdustin_trace.so")


def build(verbose=False, trace=False):
    """Compile every source and link libdustin.so; returns its path.  With
    trace=True, the phase-trace build instead (libdustin_trace.so: the same
    sources with DUSTIN_ATTN_TRACE, see include/dustin_trace.h)."""
    build_dir = BUILD + ("_trace" if trace else "")
    lib = TRACE_LIB if trace else LIB
    extra = ("-DDUSTIN_ATTN_TRACE",) if trace else ()
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, trace="--trace" in sys.argv[1:]))
