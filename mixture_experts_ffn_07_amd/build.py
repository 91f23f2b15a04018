"""Build the gfx950 shared library libmoe_mi355x.so in-tree with hipcc.

    python mixture_experts_ffn_07_amd/build.py [-v]

(run as a file: importing the package loads the built library, so it cannot
come first.)

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection switched off, then linked into one shared object next to this file.
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
OUT_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(OUT_DIR, "libmoe_mi355x.so")
SOURCES = ["abi.cpp", "route.hip", "decode.hip", "batched.hip", "gemm_large.hip", "backward.hip",
           "scratch.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-mcode-object-version=5",
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include")]


def _compile(src: str, obj: str, verbose: bool) -> None:
    lang = ["-x", "hip"] if src.endswith((".hip", ".cpp")) else []
    cmd = [hipcc()] + COMMON + lang + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{msg}")
    if verbose and msg.strip():
        print(msg, flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libmoe_mi355x.so."""
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = []
        for s in SOURCES:
            obj = os.path.join(OUT_DIR, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, os.path.join(CSRC, s), obj, verbose))
        for f in futs:
            f.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
