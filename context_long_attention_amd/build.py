"""Build libcpattn.so in-tree with hipcc for gfx950.

Usage: ``python -m context_long_attention_amd.build`` (or ``build()`` from Python).
Every call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcpattn.so")
SOURCES = ["host.cpp", "attn_fwd.hip", "attn_bwd.hip", "merge.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libcpattn")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    outdir = os.path.join(PKG, "_build")
    os.makedirs(outdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [hipcc, *lang, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "packed-fp32-ops' is not a recognized feature"
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
