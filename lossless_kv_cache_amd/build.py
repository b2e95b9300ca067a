"""Build libskv.so in-tree with hipcc for gfx950.

Usage: ``python -m lossless_kv_cache_amd.build`` (or ``build()`` from Python).
The library is placed next to this file so that it travels with the tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libskv.so")
ARCH = os.environ.get("SKV_OFFLOAD_ARCH", "gfx950")


def _hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libskv")


COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Wno-unused-parameter"]
# the HIP sources: gfx950 code with no packed FP32 instructions
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def device_asm(out: str) -> str:
    """Write the gfx950 assembly of the kernels, compiled as the library
    compiles them, to `out` (for static checks of the generated code)."""
    subprocess.check_call([_hipcc(), *DEVICE, *COMMON, "--cuda-device-only", "-S",
                           os.path.join(CSRC, "skv_kernels.hip"), "-o", out])
    return out


def build(verbose: bool = False) -> str:
    """Compile every source (always; this is the build check)."""
    hipcc = _hipcc()
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src, device in (("skv_fit.cpp", False), ("skv_api.cpp", False), ("skv_store.cpp", False),
                        ("skv_kernels.hip", True)):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
        if device:
            cmd[1:1] = DEVICE
        else:
            cmd[1:1] = ["-ffp-contract=off", "-D__HIP_PLATFORM_AMD__"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    link = [hipcc, "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
