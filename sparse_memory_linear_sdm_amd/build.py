"""Build libsdm.so (hand-written HIP kernels for gfx950 + the C ABI) in-tree.

    python -m sparse_memory_linear_sdm_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsdm.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "select.hip", "scan.hip", "init.hip", "decode.hip", "backward.hip",
           "scratch.hip", "project.hip", "scan_planned.hip"]
HIPCC = "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        # hipcc's host pass does not know the gfx-only feature flag; that note is harmless.
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
        if msg.strip() and verbose:
            print(msg)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
