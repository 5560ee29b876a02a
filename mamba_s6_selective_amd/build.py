"""Builds libssmscan.so (HIP, gfx950) in place, next to this file.

    python -m mamba_s6_selective_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libssmscan.so"
SOURCES = ["ssmscan.cpp", "linear_scan.hip", "linear_3pass.hip", "s6_scan.hip"]

# Packed-FP32 instructions are switched off for every HIP source; the
# compiler otherwise forms them on its own from scalar float code.
HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def build(verbose: bool = False) -> Path:
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), *HIPCC_FLAGS, *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libssmscan.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
