"""Build the HIP library ``lib/libkvcache.so`` for gfx950, in-tree.

Every source under ``csrc/`` is compiled by hipcc for the MI355X (gfx950)
only, then linked into one shared library with a C ABI (``include/kvcache.h``).
The measurement helper under ``measure/`` (a plain read of a decode launch's
pages, the benchmark's roofline reference) becomes ``lib/libkvmeasure.so``.
Packed-fp32 VALU instructions are disabled: the kernels rely on ordinary fp32,
packed fp16 and MFMA arithmetic.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_DIR = os.path.join(HERE, "lib")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(LIB_DIR, "libkvcache.so")
MEASURE_DIR = os.path.join(HERE, "measure")
MEASURE_LIB_PATH = os.path.join(LIB_DIR, "libkvmeasure.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def sources(folder: str = CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    libs = [(LIB_PATH, sources(CSRC)), (MEASURE_LIB_PATH, sources(MEASURE_DIR))]
    cmds, objs = [], {}
    for lib, srcs in libs:
        objs[lib] = []
        for src in srcs:
            obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
            objs[lib].append(obj)
            cmds.append([HIPCC, *CFLAGS, "-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, r in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd))
                sys.stdout.write(r.stderr)
    for lib, _ in libs:
        tmp = lib + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs[lib]])
        os.replace(tmp, lib)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
