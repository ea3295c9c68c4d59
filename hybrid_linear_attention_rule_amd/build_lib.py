"""Build libkda.so, the KDA mixer's C-ABI library, for gfx950 with hipcc.

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection turned off (-packed-fp32-ops), and linked into one shared library
next to this file.  The library links the HIP runtime and nothing else.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkda.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["kda_api.cpp", "kda_token.hip", "kda_state.hip", "kda_prefill.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-munsafe-fp-atomics"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
