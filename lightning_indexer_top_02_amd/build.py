"""Build libcsa_indexer.so (gfx950) in-tree with hipcc.

    python -m lightning_indexer_top_02_amd.build      # or build() from Python

The HIP sources and the C ABI are compiled into one shared library placed
next to this file; the Python binding loads it from there.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa_indexer.so")
SOURCES = ["csa_kernels.hip", "csa_api.cpp"]
# measurement aid for the benchmark (a plain streaming read), not part of the ABI
CALIB_LIB = os.path.join(HERE, "libcsa_calib.so")
CALIB_SOURCES = ["csa_calib.hip"]
ARCH = os.environ.get("CSA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the CSA indexer library)")


def command(out: str = LIB, sources=SOURCES) -> list:
    srcs = [os.path.join(CSRC, s) for s in sources]
    return [
        hipcc(), "-O3", "-std=c++17", "-fPIC", "-shared",
        f"--offload-arch={ARCH}",
        # keep the compiler from forming packed-FP32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
        "-I", os.path.join(ROOT, "include"),
        "-o", out, *srcs,
    ]


def _compile(out: str, sources, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = command(tmp, sources)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    noise = "is not a recognized feature for this target"
    for line in (res.stdout + res.stderr).splitlines():
        if line.strip() and noise not in line and verbose:
            print(line)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    _compile(LIB, SOURCES, verbose)
    _compile(CALIB_LIB, CALIB_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
