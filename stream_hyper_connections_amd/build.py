"""Build libmhc.so in-tree for gfx950 with hipcc.

``python -m stream_hyper_connections_amd.build`` or ``build()`` from Python.
The flags disable packed-fp32 instruction selection on the device side.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "mhc.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmhc.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, src, "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}) building {lib}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _compile(SRC, LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
