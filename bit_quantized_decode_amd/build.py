"""Build libbqd.so (HIP kernels for gfx950 + the C ABI) in-tree.

The validation unit is plain C++ compiled with g++ (no HIP headers), the
kernels and entry points are compiled with hipcc for gfx950 only, and the
objects are linked into ``bit_quantized_decode_amd/libbqd.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libbqd.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIP_SOURCES = ["cq.hip", "f8.hip", "i8.hip", "mlp.hip", "sample.hip", "stream.hip", "capi.hip"]
HOST_SOURCES = ["validate.cpp"]
ARCH = "gfx950"
# Packed fp32 VALU instructions are turned off for every device pass.
# -disable-promote-alloca-to-lds: private arrays stay in registers; moved to
# LDS they would silently raise a kernel's LDS size and cut its occupancy.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-disable-promote-alloca-to-lds", f"-I{INCLUDE}"]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{INCLUDE}"]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libbqd.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([_hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose:
                sys.stderr.write(r.stderr)
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB_PATH + ".tmp"
    _run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
