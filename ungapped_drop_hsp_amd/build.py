"""Build libhspz.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python ungapped_drop_hsp_amd/build.py

Run it by path: importing the package itself requires the library to exist already.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhspz.so")
ARCH = os.environ.get("HSPZ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    f"--offload-arch={ARCH}",
    # Packed-FP32 VALU forms stay off: only scalar and packed-integer code is wanted.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libhspz)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    out_tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libhspz.so")
    noisy = [l for l in (res.stdout + res.stderr).splitlines()
             if "packed-fp32-ops" not in l and l.strip()]
    if noisy and verbose:
        sys.stderr.write("\n".join(noisy) + "\n")
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
