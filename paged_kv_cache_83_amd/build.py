"""Build libpa.so in place: hipcc for the gfx950 kernels, g++ for the host code.

    python paged_kv_cache_83_amd/build.py             # libpa.so
    python paged_kv_cache_83_amd/build.py --sanitize  # libpa_asan.so

(Run it as a script, or load it by path: importing the package loads the
library, which is what this file produces.)

The sanitized variant compiles the host-only C++ (block manager, radix cache)
with AddressSanitizer and UndefinedBehaviorSanitizer (g++, host code only; the
kernel sources are built as usual) for the CPU tests: load it with PA_LIB
pointing at it and the ASan runtime preloaded.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
LIB_ASAN = os.path.join(PKG, "libpa_asan.so")

ARCH = "gfx950"
# Packed-fp32 instructions are kept out of every kernel (the compiler would
# otherwise form v_pk_* fp32 ops from plain float code).
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-g"]


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


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source under csrc/ (in parallel) and link
    paged_kv_cache_83_amd/libpa.so, or libpa_asan.so with sanitize=True."""
    hipcc = _hipcc()
    cxx = os.environ.get("CXX", shutil.which("g++") or "g++")
    out_lib = LIB_ASAN if sanitize else LIB
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        jobs = []
        for name in sorted(os.listdir(CSRC)):
            src = os.path.join(CSRC, name)
            obj = os.path.join(tmp, name + ".o")
            if name.endswith(".hip"):
                jobs.append(([hipcc, *HIP_FLAGS, "-c", src, "-o", obj], obj))
            elif name.endswith(".cpp"):
                jobs.append(([cxx, *CXX_FLAGS, *(SAN_FLAGS if sanitize else []), "-c", src, "-o", obj],
                             obj))
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, cmd, verbose) for cmd, _ in jobs]:
                f.result()
        objs = [obj for _, obj in jobs]
        tmp_lib = out_lib + ".tmp"
        if sanitize:
            rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
            _run([cxx, "-shared", "-fPIC", *SAN_FLAGS, *objs, f"-L{rocm}/lib", "-lamdhip64",
                  f"-Wl,-rpath,{rocm}/lib", "-o", tmp_lib], verbose)
        else:
            _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib], verbose)
        os.replace(tmp_lib, out_lib)
    return out_lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
