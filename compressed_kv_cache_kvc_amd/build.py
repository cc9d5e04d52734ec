"""Build libkvc.so (HIP kernels + C ABI) in-tree for gfx950.

    python compressed_kv_cache_kvc_amd/build.py

Compiles every source under csrc/ with hipcc (host-only C++ with g++) into
``_build/`` and links ``compressed_kv_cache_kvc_amd/libkvc.so``. No fast-math:
the quantizer relies on correctly rounded fp32 division and round-half-even.
Packed fp32 instructions are disabled in device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvc.so")
ARCH = os.environ.get("KVC_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", f"-I{INCLUDE}"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def build_library(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src) + ".o")
        if src.endswith(".hip"):
            cmd = [hipcc, *HIP_FLAGS, *extra_flags, "-c", src, "-o", obj]
        else:
            cmd = ["g++", *CXX_FLAGS, "-c", src, "-o", obj]
        jobs.append((cmd, obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for (cmd, _), r in zip(jobs, ex.map(lambda j: _run(j[0]), jobs)):
            if verbose:
                print(" ".join(cmd))
                sys.stdout.write(r.stderr)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for _, o in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
