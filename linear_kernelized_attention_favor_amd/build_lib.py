"""Build libfavor.so in-tree with hipcc for gfx950.

Usage: python linear_kernelized_attention_favor_amd/build_lib.py [-v]
(this file imports nothing from the package, so it runs before a library exists)

Every source under csrc/ is compiled to an object in csrc/_build/ (in
parallel), then linked into linear_kernelized_attention_favor_amd/libfavor.so.
HIP sources (.hip) are compiled for gfx950 only; host sources (.cpp) are
compiled by hipcc as plain C++ against the HIP headers.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libfavor.so")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
# Keep packed fp32 arithmetic out of the device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfavor.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), "-x", "hip", *DEVICE, *COMMON, "-c", src, "-o", obj]
    else:
        # Host-only C++: the system compiler against the HIP headers.
        cmd = [shutil.which("g++") or "g++", *COMMON, "-D__HIP_PLATFORM_AMD__",
               f"-I{os.path.join(rocm(), 'include')}", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so.
    err = "\n".join(l for l in r.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
