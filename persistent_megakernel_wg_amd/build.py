"""Build libmk.so (the decode megakernel and its C ABI) in-tree for gfx950.

    python -m persistent_megakernel_wg_amd.build

The kernel is compiled by hipcc for gfx950 only; the planner is plain C++ and
the runtime is C++ against the HIP host API.  Packed-fp32 instructions are
disabled for device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmk.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-I", os.path.join(ROOT, "include")]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
              "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l
                    and "reserved registers" not in l)
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, extra_defines=()) -> str:
    """Compile every source and link libmk.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    gxx = shutil.which("g++") or "g++"
    defs = ["-D" + d for d in extra_defines]
    k_obj = os.path.join(BUILD, "mk_kernel.o")
    p_obj = os.path.join(BUILD, "mk_plan.o")
    r_obj = os.path.join(BUILD, "mk_runtime.o")
    b_obj = os.path.join(BUILD, "mk_batch.o")
    s_obj = os.path.join(BUILD, "mk_static.o")
    d_obj = os.path.join(BUILD, "mk_diag.o")
    _run([hipcc, *DEVICE_FLAGS, *defs, "-c", os.path.join(CSRC, "mk_kernel.hip"), "-o", k_obj], verbose)
    _run([hipcc, *DEVICE_FLAGS, *defs, "-c", os.path.join(CSRC, "mk_batch.hip"), "-o", b_obj], verbose)
    _run([hipcc, *DEVICE_FLAGS, *defs, "-c", os.path.join(CSRC, "mk_static.hip"), "-o", s_obj], verbose)
    _run([hipcc, *DEVICE_FLAGS, *defs, "-c", os.path.join(CSRC, "mk_diag.hip"), "-o", d_obj], verbose)
    _run([gxx, *HOST_FLAGS, "-c", os.path.join(CSRC, "mk_plan.cpp"), "-o", p_obj], verbose)
    _run([gxx, *HOST_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-c", os.path.join(CSRC, "mk_runtime.cpp"), "-o", r_obj], verbose)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", k_obj, b_obj, s_obj, d_obj, p_obj, r_obj,
          "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
