"""Compile libpkm.so (HIP, gfx950 only) in place with hipcc.

    python -m product_key_memory_amd.build
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
LIB_PATH = os.path.join(PKG, "libpkm.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpkm.so)")


def build_library(out: str = LIB_PATH, verbose: bool = False, defines: tuple = (),
                  csrc: str = CSRC) -> str:
    sources = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-munsafe-fp-atomics",
        # packed float32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", csrc, *[f"-D{d}" for d in defines], *sources, "-o", out + ".tmp",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
