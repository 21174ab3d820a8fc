"""Build ``libsparsepr.so`` (the HIP C-ABI library) for gfx950 with hipcc.

Sources are compiled to position-independent objects under ``_build/`` at the
repository root and linked into ``free_block_sparse_rcp_amd/lib/``. Run as
``python -m free_block_sparse_rcp_amd.build``; it always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libsparsepr.so"
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["api.hip", "partition.hip", "route.hip", "attention.hip", "fit.hip", "apply.hip",
           "support.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = lib_path() + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    # a kernel whose host stub was not instantiated links fine and fails at dlopen
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r})"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"built library does not load:\n{r.stderr}")
    os.replace(tmp, lib_path())
    if verbose:
        print(f"built {lib_path()}")
    return lib_path()


if __name__ == "__main__":
    build()
