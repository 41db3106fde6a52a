"""Compile libpkm.so (HIP, gfx950 only) in place with hipcc.

    python -m product_key_memory_amd.build [--incremental]

Each source is compiled to an object of its own, all in parallel, and the
objects are linked into the shared library.  With ``incremental`` an object is
reused when its source, the headers and the flags are unchanged (a digest of
them names the object); the default rebuilds everything.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libpkm.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    # packed float32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpkm.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {cmd[-1]}")


def _local_includes(path: str, dirs, seen=None) -> list:
    """Files reached through #include "..." from `path`, searched in `dirs`."""
    seen = set() if seen is None else seen
    with open(path, encoding="utf-8") as fh:
        names = re.findall(r'^\s*#\s*include\s*"([^"]+)"', fh.read(), re.M)
    for name in names:
        for d in [os.path.dirname(path), *dirs]:
            cand = os.path.join(d, name)
            if os.path.exists(cand) and cand not in seen:
                seen.add(cand)
                _local_includes(cand, dirs, seen)
                break
    return sorted(seen)


def build_library(out: str = LIB_PATH, verbose: bool = False, defines: tuple = (),
                  csrc: str = CSRC, incremental: bool = False) -> str:
    sources = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    flags = FLAGS + ["-I", INCLUDE, "-I", csrc, *[f"-D{d}" for d in defines]]
    obj_dir = OBJ_DIR if out == LIB_PATH else os.path.join(os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    objects = []
    for src in sources:
        d = hashlib.sha256(" ".join(flags).encode())
        for f in [src, *_local_includes(src, [csrc, INCLUDE])]:
            with open(f, "rb") as fh:
                d.update(fh.read())
        obj = os.path.join(obj_dir, f"{os.path.basename(src)}.{d.hexdigest()[:16]}.o")
        objects.append(obj)
        if not (incremental and os.path.exists(obj)):
            jobs.append([hipcc(), *flags, "-c", src, "-o", obj + ".tmp"])
    workers = min(len(jobs), max(1, os.cpu_count() or 1)) or 1
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for fut in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
            fut.result()
    for cmd in jobs:
        os.replace(cmd[-1], cmd[-1][:-4])
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objects, "-o", out + ".tmp"],
         verbose)
    os.replace(out + ".tmp", out)
    keep = set(objects)
    for old in glob.glob(os.path.join(obj_dir, "*.o")):
        if old not in keep:
            os.remove(old)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True, incremental="--incremental" in sys.argv))
