"""Build libfa355.so (and the microbenchmark library libfa355_mb.so) in-tree with hipcc for gfx950.

Usage: ``python tiled_attention_06_amd/build.py`` (or ``__graft_entry__.build()``).
This file is run as a script or loaded by path: importing the package itself
requires the library to exist already.
The library is written next to this file; a temporary name plus an atomic
rename keeps a half-written library from ever being loaded.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa355.hip")
OUT = os.path.join(PKG, "libfa355.so")
# microbenchmarks of the units (bench.py --microbench): a library of its own, never loaded by the package
MB_SRC = os.path.join(PKG, "csrc", "microbench.hip")
MB_OUT = os.path.join(PKG, "libfa355_mb.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs where they are used by VALU code: without it the dK/dV
    # kernel (one wave per SIMD, over 256 registers) put its score tiles in AGPRs and
    # copied every element back (~9 VALU copies per MFMA); the other kernels'
    # machine code is unchanged by it
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
    "-Wl,--no-undefined",  # a missing kernel stub must fail the build, not the first load
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa355)")


def build_library(out: str = OUT, verbose: bool = False, src: str = SRC) -> str:
    tmp = f"{out}.tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list[str]:
    """Every HIP library of the package: libfa355.so and the microbenchmarks' libfa355_mb.so."""
    return [build_library(OUT, verbose, SRC), build_library(MB_OUT, verbose, MB_SRC)]


if __name__ == "__main__":
    for path in build_all(verbose="-v" in sys.argv):
        print(path)
