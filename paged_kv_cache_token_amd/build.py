"""Build libpa.so (the paged-attention C ABI) for gfx950 with hipcc, in-tree.

    python paged_kv_cache_token_amd/build.py     (by path: the package itself
                                                 loads libpa.so on import)

compiles every csrc/*.hip file (hipcc, gfx950) and every host-only csrc/*.cpp
file (g++) to an object under _build/, in parallel, and links them into
paged_kv_cache_token_amd/libpa.so.  It always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 math.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
]


CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE]


def _cxx() -> str:
    exe = shutil.which("g++") or shutil.which("c++")
    if not exe:
        raise RuntimeError("no host C++ compiler (g++) found")
    return exe


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libpa.so")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature: harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    host_sources = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))  # host-only C++
    objects = [os.path.join(BUILD_DIR, os.path.basename(s) + ".o") for s in sources + host_sources]
    cmds = [[hipcc, *HIP_FLAGS, "-c", s, "-o", o] for s, o in zip(sources, objects)]
    cmds += [[_cxx(), *CXX_FLAGS, "-c", s, "-o", o]
             for s, o in zip(host_sources, objects[len(sources):])]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, c, verbose) for c in cmds]
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objects], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
