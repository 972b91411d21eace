"""Build libfa.so (the C-ABI attention library) in-tree for gfx950 with hipcc.

    python -m exact_io_aware_56_amd.build        # from the repository root

Produces exact_io_aware_56_amd/libfa.so; intermediate objects go to
exact_io_aware_56_amd/_build/. Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa)")
    return exe


def run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(extra_flags=(), lib: str = LIB, obj_dir: str = OUT_DIR) -> str:
    """Compile and link libfa.so. `extra_flags` (e.g. -DFA_KEY_TILE=32) reach
    the kernel compile only; `lib` / `obj_dir` redirect the outputs."""
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    kern_o = os.path.join(obj_dir, "fa_fwd.o")
    api_o = os.path.join(obj_dir, "fa_api.o")
    run([cc, f"--offload-arch={ARCH}", *COMMON, *DEVICE_FLAGS, *extra_flags, "-x", "hip", "-c",
         os.path.join(CSRC, "fa_fwd.hip"), "-o", kern_o])
    run([cc, *COMMON, "-c", os.path.join(CSRC, "fa_api.cpp"), "-o", api_o])
    tmp = lib + ".tmp"
    # -z defs: an unresolved symbol (e.g. a kernel handle the host pass failed
    # to emit) fails the link instead of the first dlopen
    run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", kern_o, api_o, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
