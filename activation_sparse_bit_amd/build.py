"""Compile the HIP library ``lib/libsgemv.so`` (and the measurement-only
``lib/libsgemv_bench.so``) in-tree for gfx950.

The host packer (pack.cpp) is plain C++ built with g++; the kernels and the
C ABI (sgemv.hip) are built with hipcc for gfx950.  All HIP code is
compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libsgemv.so")
BENCH_LIB = os.path.join(LIBDIR, "libsgemv_bench.so")   # measurement-only read kernels

HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    obj_dir = os.path.join(LIBDIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    pack_o = os.path.join(obj_dir, "pack.o")
    sgemv_o = os.path.join(obj_dir, "sgemv.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-c",
          os.path.join(CSRC, "pack.cpp"), "-o", pack_o], verbose)
    _run([_hipcc(), *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, "sgemv.hip"),
          "-o", sgemv_o], verbose)
    tmp = LIB + ".tmp"
    _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", sgemv_o, pack_o,
          "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # the measurement kernels (memory ceilings), a library of their own
    bench_o = os.path.join(obj_dir, "bench_read.o")
    _run([_hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, "bench_read.hip"), "-o", bench_o], verbose)
    tmp = BENCH_LIB + ".tmp"
    _run([_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", bench_o, "-o", tmp], verbose)
    os.replace(tmp, BENCH_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
