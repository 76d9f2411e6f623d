"""Build libpa.so in place: hipcc for the gfx950 kernels, g++ for the host code.

    python paged_kv_cache_83_amd/build.py

(Run it as a script, or load it by path: importing the package loads the
library, which is what this file produces.)
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")

ARCH = "gfx950"
# Packed-fp32 instructions are kept out of every kernel (the compiler would
# otherwise form v_pk_* fp32 ops from plain float code).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source under csrc/ and link paged_kv_cache_83_amd/libpa.so."""
    hipcc = _hipcc()
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        objs = []
        for name in sorted(os.listdir(CSRC)):
            src = os.path.join(CSRC, name)
            obj = os.path.join(tmp, name + ".o")
            if name.endswith(".hip"):
                _run([hipcc, *HIP_FLAGS, "-c", src, "-o", obj], verbose)
            elif name.endswith(".cpp"):
                _run([cxx, *CXX_FLAGS, "-c", src, "-o", obj], verbose)
            else:
                continue
            objs.append(obj)
        tmp_lib = LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
