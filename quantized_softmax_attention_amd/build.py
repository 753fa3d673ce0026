"""Build libkia.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m quantized_softmax_attention_amd.build

Objects go to ``_build/`` at the repository root; the shared library lands
next to this file, where the binding loads it from.
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
LIB = os.path.join(PKG, "libkia.so")
SOURCES = ["kia_api.hip", "kia_forward.hip", "kia_backward.hip", "kia_p1.hip", "kia_geometry.hip"]
# the benchmark's matrix-core peak probe: a separate library, no part of libkia
PEAK_LIB = os.path.join(PKG, "libkia_peak.so")
PEAK_SOURCE = "kia_peak.hip"

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkia")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    peak_tmp = PEAK_LIB + ".tmp"
    cmds.append([cc, *HIPCC_FLAGS, "-shared", os.path.join(CSRC, PEAK_SOURCE), "-o", peak_tmp])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    os.replace(peak_tmp, PEAK_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
