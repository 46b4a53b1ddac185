"""Compile the HIP library libmuon_mi355x.so for gfx950, in-tree.

    python -m muon_newton_schulz_step_amd.build

Each source is compiled to an object under _build/ (in parallel), then linked
into the package directory, where the Python binding loads it from.
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
LIB_NAME = "libmuon_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["plan.cpp", "abi.cpp", "noalloc.hip", "k_elem.hip", "k_gemm.hip", "k_gemm256.hip", "k_head.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {LIB_NAME} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
