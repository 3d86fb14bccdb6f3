"""Build libdsv4.so (the C-ABI library) in-tree with hipcc for gfx950.

    python sparse_mla_attention_combine_amd/build.py [--verbose]

Every source is compiled to an object in parallel, then linked into
``sparse_mla_attention_combine_amd/_lib/libdsv4.so``.  hipcc cross-compiles, so this
runs on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(OUT_DIR, "libdsv4.so")
ARCH = "gfx950"
SOURCES = ["api.cpp", "combine.hip", "insert.hip", "gather.hip", "attention.hip",
           "workspace.hip", "indexer.hip", "peaks.hip"]
# Packed FP32 instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Wno-unused-result", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose and src.endswith(".hip"):
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "unknown target feature" not in l and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{msg}")
    if verbose and msg.strip():
        print(f"--- {src}\n{msg}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
