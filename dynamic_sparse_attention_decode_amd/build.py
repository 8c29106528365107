"""Build libprr.so (HIP for gfx950) in-tree: ``python -m dynamic_sparse_attention_decode_amd.build``.

Every .hip source is compiled for gfx950 only; the host-only budget chooser is plain C++. Object files go to
``_build/`` at the repository root and the library to ``dynamic_sparse_attention_decode_amd/lib/libprr.so``.
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
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libprr.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIP_SOURCES = ["prr_api.hip", "summaries.hip", "select.hip", "attend.hip", "fused.hip", "two_launch.hip"]
CXX_SOURCES = ["budget.cpp"]

# Packed fp32 ops are switched off for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libprr.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    hipcc = _hipcc()
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmds.append([hipcc, "-O2", "-std=c++17", "-fPIC", "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for c, o in zip(cmds, outs):
            print(" ".join(c))
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
