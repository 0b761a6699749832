"""Builds libdsa.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Usage: python dsa_sparse_attention_indexer_amd/build.py
(run as a file: importing the package itself loads the library this script builds)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["api.hip", "indexer.hip", "topk.hip", "block_select.hip", "sparse_mla.hip", "cache_insert.hip"]
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")
# Packed fp32 instructions are kept out of generated code (plain scalar fp32 only).
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _quiet(out: str) -> str:
    # hipcc's host pass does not know the packed-fp32 target feature; that warning is harmless
    return "\n".join(l for l in out.splitlines() if "not a recognized feature" not in l)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc, *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msg = _quiet(r.stdout + r.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{_quiet(r.stdout + r.stderr)}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
