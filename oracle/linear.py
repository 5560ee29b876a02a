"""Float64 oracle for the first-order linear recurrence (test infrastructure).

Source: "Selective-scan CUDA kernels" (persus.netlify.app/projects/selective-scan),
the paragraph stating h[t] = a[t]*h[t-1] + b[t] and its reading as a prefix scan
over affine pairs (associative, not commutative).

Readings of what the page leaves open:
* indexing: h[-1] = h0 is the carry-in, so h[0] = a[0]*h0 + b[0]; every h[t]
  (the inclusive prefix) is returned.
* pair order: (a1, b1) (+) (a2, b2) composes the earlier map (a1, b1) first,
  giving (a1*a2, a2*b1 + b2).
"""
from __future__ import annotations

import numpy as np


def linear_scan(a, b, h0: float = 0.0) -> np.ndarray:
    """h[t] = a[t]*h[t-1] + b[t] with h[-1] = h0, sequentially, in float64.

    Plain Python loop over Python floats: meant for n up to ~1e6. Larger inputs
    go through ``oracle.native.linear_scan``.
    """
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    if a.shape != b.shape:
        raise ValueError("a and b must have the same length")
    out = np.empty(a.shape[0], dtype=np.float64)
    h = float(h0)
    al = a.tolist()
    bl = b.tolist()
    for t in range(len(al)):
        h = al[t] * h + bl[t]
        out[t] = h
    return out


def affine_combine(p, q):
    """Compose two affine maps, earlier map ``p`` first: x -> q(p(x)).

    p = (a1, b1) is x -> a1*x + b1 and q = (a2, b2) is x -> a2*x + b2, so
    q(p(x)) = a2*(a1*x + b1) + b2 = (a1*a2)*x + (a2*b1 + b2).
    Works on Python floats, numpy scalars or fractions.Fraction alike.
    """
    a1, b1 = p
    a2, b2 = q
    return (a1 * a2, a2 * b1 + b2)


def apply_affine(p, x):
    """Evaluate the affine map p = (a, b) at x."""
    a, b = p
    return a * x + b


def affine_prefix(a, b):
    """Inclusive prefix of the affine maps (a[t], b[t]) by a left fold.

    Returns a list of pairs P[t] = (...((m0 (+) m1) (+) m2) ... (+) m_t); the
    recurrence value is h[t] = apply_affine(P[t], h0).
    """
    out = []
    acc = None
    for at, bt in zip(a, b):
        m = (at, bt)
        acc = m if acc is None else affine_combine(acc, m)
        out.append(acc)
    return out
