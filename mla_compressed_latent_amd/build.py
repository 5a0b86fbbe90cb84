"""Build the HIP library libmla.so in-tree with hipcc for gfx950.

    python mla_compressed_latent_amd/build.py [--verbose]

(run by path: importing the package loads the library this script builds)

Each source compiles to an object under ``_build/`` in parallel; the objects
are linked into ``mla_compressed_latent_amd/libmla.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "pack.hip", "append.hip", "gemm_heads.hip", "splitkv.hip", "splitkv_x8.hip", "splitkv_r128.hip",
           "extend.hip", "project.hip", "check.hip", "pool.cpp"]
# The checking build (libmla_debug.so): the same objects, with api.hip
# compiled again with MLA_DEBUG_CHECKS (device-resident lengths and page ids
# verified before each call's kernels run).
DEBUG_LIB = os.path.join(PKG, "libmla_debug.so")
DEBUG_SOURCE = "api.hip"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla.so)")


def _compile(src: str, verbose: bool, debug: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ("_debug.o" if debug else ".o"))
    cmd = [hipcc(), *HIPCC_FLAGS, *(["-DMLA_DEBUG_CHECKS=1"] if debug else []), "-I", os.path.join(ROOT, "include"),
           "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs and verbose:
        print(errs, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Build libmla.so and the checking build libmla_debug.so; returns the former's path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(DEBUG_SOURCE, True)]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    release = objs[:len(SOURCES)]
    debug = [objs[-1] if s == DEBUG_SOURCE else o for s, o in zip(SOURCES, release)]
    _link(release, LIB, verbose)
    _link(debug, DEBUG_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
