"""Build libmoe.so (the HIP kernels + the C ABI) in-tree for gfx950.

    python -m sparse_mixture_experts_28_amd.build

compiles every source under csrc/ with hipcc --offload-arch=gfx950 into
_build/ and links sparse_mixture_experts_28_amd/libmoe.so.  It always
recompiles (it is the build check).  hipcc cross-compiles, so no GPU is needed.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

SOURCES = ["router.hip", "permute.hip", "expert_choice.hip", "gemm.hip", "mxfp8.hip", "combine.hip", "moe_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if r.stderr.strip():
        warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
        if warn.strip():
            print(f"[build] {src}:\n{warn}", file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # a library can link and still not load: refuse one that leaves any of
    # this project's symbols undefined (hipcc's host pass has been seen to
    # drop a kernel's launch stub while still referencing it)
    r = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines() if "_ZN3moe" in l]
    if r.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("libmoe.so would not load; undefined: " + (", ".join(missing) or r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print(f"[build] wrote {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
