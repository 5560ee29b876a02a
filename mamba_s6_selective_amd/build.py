"""Builds libssmscan.so (HIP, gfx950) in place, next to this file.

    python -m mamba_s6_selective_amd.build [--force]

Each source compiles to an object in parallel; the objects are then linked
into the shared library, which replaces the old one only once complete.
Objects are kept in _build/ under a hash of the source, every header of
csrc/ and include/, and the flags, and reused when nothing changed, unless
force is set (build(force=True) always compiles every source).
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
CSRC = PKG / "csrc"
LIB = PKG / "libssmscan.so"
CACHE = PKG / "_build"
SOURCES = ["ssmscan.cpp", "linear_scan.hip", "linear_3pass.hip", "s6_scan.hip"]

# Packed-FP32 instructions are switched off for every HIP source; the
# compiler otherwise forms them on its own from scalar float code.
HIPCC_FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-fPIC", "-shared"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = Path(rocm) / "bin" / "hipcc"
    return str(cand) if cand.exists() else "hipcc"


def _key(src: str) -> str:
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    h.update((CSRC / src).read_bytes())
    for hdr in sorted(list(CSRC.glob("*.h")) + list((PKG.parent / "include").glob("*.h"))):
        h.update(hdr.name.encode())
        h.update(hdr.read_bytes())
    return h.hexdigest()[:20]


def build(verbose: bool = False, force: bool = False) -> Path:
    CACHE.mkdir(exist_ok=True)
    work = Path(tempfile.mkdtemp(prefix="ssmscan_build_"))
    try:
        objs, procs = [], []
        for src in SOURCES:
            cached = CACHE / f"{Path(src).stem}.{_key(src)}.o"
            if cached.exists() and not force:
                objs.append(cached)
                continue
            obj = work / (Path(src).stem + ".o")
            objs.append(obj)
            cmd = [hipcc(), *HIPCC_FLAGS, "-c", str(CSRC / src), "-o", str(obj)]
            procs.append((src, obj, cached, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                             stderr=subprocess.PIPE, text=True)))
        failed = False
        for src, obj, cached, p in procs:
            out, err = p.communicate()
            if p.returncode != 0:
                sys.stderr.write(f"--- {src}\n{out}{err}")
                failed = True
            else:
                if verbose:
                    sys.stderr.write(err)
                for old in CACHE.glob(f"{Path(src).stem}.*.o"):
                    old.unlink()
                shutil.copyfile(obj, cached)
        if failed:
            raise RuntimeError("hipcc failed building libssmscan.so")
        tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
        res = subprocess.run([hipcc(), *LINK_FLAGS, *map(str, objs), "-o", str(tmp)],
                             capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libssmscan.so")
        os.replace(tmp, LIB)
        return LIB
    finally:
        shutil.rmtree(work, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=True, force="--force" in sys.argv[1:]))
