"""Float64 oracle for the S6 selective scan (test infrastructure).

Sources:
* POPCORNBENCH transcript FW-GLM-5-1 (level 2, problem 30), the problem
  statement's forward pass: delta (B, L, D), B_t and C_t (B, L, N), A = -exp(A_log)
  (D, N); dA = exp(delta*A) and dB = delta*B_t with broadcasting to (B, L, D, N);
  x_db = x*dB; at each step h = dA[:, t]*h + x_db[:, t] and y_t = sum_n h*C_t; the
  output is y + x*D. Its sequential kernel sketch starts h at zero and writes
  y[b, t, d] after updating h at step t.
* "ARM-Scan — Optimized Mamba Selective-Scan Kernel", sections "Approach" and
  "What broke": a reverse recurrence that shares the forward one's discretized
  terms, fused with it, and equal to two independent scans.

* The same transcript's model computes delta = softplus(proj_delta(x)), the
  projection carrying a bias, with softplus(x) = log(1 + exp(x)) evaluated by
  the log1p-exp trick.

Readings (where the pages are silent):
* u is the transcript's x; by default delta is passed after softplus and used
  as given. With delta_softplus=True the scan applies softplus to
  delta + delta_bias[d] itself (the bias being the projection's, added before
  the softplus); delta_bias alone (without softplus) is not a form the pages
  use and is rejected.
* reverse: h_r[L] = 0 and h_r[t] = dA[t]*h_r[t+1] + x_db[t] for t = L-1 .. 0,
  with the same dA[t], x_db[t] as the forward pass; y_r[t] = sum_n C[t]*h_r[t] + D*u[t].
* bidirectional: y = y_fwd + y_rev, each with its own D*u term, so D*u counts
  twice and bidir == fwd + flip_L(fwd(flip_L(inputs))) holds exactly.
"""
from __future__ import annotations

import numpy as np

DIRECTIONS = ("fwd", "rev", "bidir")


def softplus(x) -> np.ndarray:
    """log(1 + exp(x)) in float64, by numpy's logaddexp(0, x) (exact for large
    |x|: no overflow for x >> 0, no cancellation for x << 0)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def _one_direction(u, delta, A, B, C, D, reverse: bool) -> np.ndarray:
    batch, L, d_inner = u.shape
    N = A.shape[1]
    h = np.zeros((batch, d_inner, N), dtype=np.float64)
    y = np.empty((batch, L, d_inner), dtype=np.float64)
    steps = range(L - 1, -1, -1) if reverse else range(L)
    for t in steps:
        dt = delta[:, t, :]                      # (batch, d)
        x = u[:, t, :]                           # (batch, d)
        dA = np.exp(dt[:, :, None] * A[None, :, :])          # (batch, d, N)
        dB = dt[:, :, None] * B[:, t, None, :]               # (batch, d, N)
        x_db = x[:, :, None] * dB                            # (batch, d, N)
        h = dA * h + x_db
        y[:, t, :] = np.sum(h * C[:, t, None, :], axis=-1) + x * D[None, :]
    return y


def selective_scan(u, delta, A, B, C, D, direction: str = "fwd", delta_bias=None,
                   delta_softplus: bool = False) -> np.ndarray:
    """S6 output y of shape (batch, L, d_inner), float64.

    u, delta: (batch, L, d_inner); A: (d_inner, N); B, C: (batch, L, N);
    D: (d_inner,); delta_bias: (d_inner,) or None. Any float dtype; everything
    is widened to float64 first. With delta_softplus, delta is replaced by
    softplus(delta + delta_bias) before the scan. Loops over t in Python and
    vectorises over (batch, d_inner, N).
    """
    if direction not in DIRECTIONS:
        raise ValueError(f"direction must be one of {DIRECTIONS}")
    if delta_bias is not None and not delta_softplus:
        raise ValueError("delta_bias is only applied together with delta_softplus")
    if delta_softplus:
        delta = np.asarray(delta, dtype=np.float64)
        if delta_bias is not None:
            delta = delta + np.asarray(delta_bias, dtype=np.float64)[None, None, :]
        delta = softplus(delta)
    u = np.asarray(u, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    batch, L, d_inner = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or A.shape != (d_inner, N) or D.shape != (d_inner,) \
            or B.shape != (batch, L, N) or C.shape != (batch, L, N):
        raise ValueError("inconsistent S6 shapes")
    if direction == "fwd":
        return _one_direction(u, delta, A, B, C, D, reverse=False)
    if direction == "rev":
        return _one_direction(u, delta, A, B, C, D, reverse=True)
    return (_one_direction(u, delta, A, B, C, D, reverse=False)
            + _one_direction(u, delta, A, B, C, D, reverse=True))
