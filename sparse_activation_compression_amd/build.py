"""Build libcdma.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""

from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcdma.so")

SOURCES = ("kernels.hip", "cdma_api.cpp", "offload.cpp", "prefetch.cpp", "pinned_pool.cpp")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise FileNotFoundError("hipcc not found (ROCm is required to build libcdma)")


def build_library(out: str = LIB, arch: str = "gfx950", extra=(), verbose: bool = False) -> str:
    """Compile every source into one shared library; returns its path."""
    cmd = [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={arch}", "-fPIC", "-shared",
        # packed fp32 instructions are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # every atomic here is issued by one lane on purpose; the wave-level
        # atomic rewrite would make the issuing wave wait for the result at once
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        *extra,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
