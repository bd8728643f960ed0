"""Build libmoe_mxfp4.so for gfx950 with hipcc (in-tree, next to this file).

    python -m mxfp4_routed_expert_route_amd.build

Compiles every source in csrc/ (object files under _build/) and links the
shared library.  Also builds the host-only check program of the argument
validation layer (g++, address and undefined-behaviour sanitizers), which
the CPU tests run.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe_mxfp4.so")
VALIDATE_CHECK = os.path.join(BUILD, "validate_check")

ARCH = "gfx950"
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions (v_pk_fma_f32 & co.)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        cmd = [hipcc, *HIP_FLAGS, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        _run(cmd)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


def build_validate_check() -> str:
    """Host-only build of validate.cpp plus a C driver, with sanitizers (no GPU)."""
    os.makedirs(BUILD, exist_ok=True)
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    _run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", os.path.join(CSRC, "validate.cpp"),
          os.path.join(CSRC, "host_check", "validate_check.cpp"), "-o", VALIDATE_CHECK])
    return VALIDATE_CHECK


def build(verbose: bool = False) -> None:
    build_library(verbose)
    build_validate_check()


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
