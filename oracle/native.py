"""ctypes loader for the plain C float64 twin of the oracle (test infrastructure).

``build()`` compiles ``oracle_c.c`` with gcc into ``liboracle.so`` beside it.
The loaders build it only when no built library is present.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SRC = _HERE / "oracle_c.c"
LIB = _HERE / "liboracle.so"

_DIRS = {"fwd": 0, "rev": 1, "bidir": 2}
_lib = None


def build() -> Path:
    """Compile the C twin (always; callers that only need it loaded use load())."""
    tmp = LIB.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-o", str(tmp), str(SRC), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not LIB.exists():
        build()
    lib = ctypes.CDLL(str(LIB))
    f = lib.oracle_linear_scan
    f.restype = None
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double,
                  ctypes.c_void_p, ctypes.c_int64]
    g = lib.oracle_s6
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 4 + \
        [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int]
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Widen to a contiguous float64 array (exact for fp32 and bf16 data)."""
    if hasattr(x, "detach"):          # torch tensor
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def linear_scan(a, b, h0: float = 0.0) -> np.ndarray:
    """h[t] = a[t]*h[t-1] + b[t], h[-1] = h0, in float64."""
    a = _f64(a).ravel()
    b = _f64(b).ravel()
    if a.shape != b.shape:
        raise ValueError("a and b must have the same length")
    h = np.empty(a.shape[0], dtype=np.float64)
    load().oracle_linear_scan(a.ctypes.data, b.ctypes.data, float(h0),
                              h.ctypes.data, a.shape[0])
    return h


def selective_scan(u, delta, A, B, C, D, direction: str = "fwd",
                   ch_begin: int = 0, ch_end: int | None = None,
                   nthreads: int = 0, out: np.ndarray | None = None):
    """S6 output (float64, (batch, L, d_inner)) and the thread count used.

    Only the flattened (batch, d_inner) channels [ch_begin, ch_end) are
    computed; the rest of ``out`` is left as it was (NaN when allocated here).
    """
    u, delta, A, B, C, D = (_f64(t) for t in (u, delta, A, B, C, D))
    batch, L, d_inner = u.shape
    N = A.shape[1]
    if ch_end is None:
        ch_end = batch * d_inner
    if out is None:
        out = np.full((batch, L, d_inner), np.nan, dtype=np.float64)
    used = load().oracle_s6(u.ctypes.data, delta.ctypes.data, A.ctypes.data,
                            B.ctypes.data, C.ctypes.data, D.ctypes.data,
                            out.ctypes.data, batch, L, d_inner, N,
                            _DIRS[direction], ch_begin, ch_end, nthreads)
    if used < 0:
        raise ValueError("oracle_s6 rejected its arguments")
    return out, used
