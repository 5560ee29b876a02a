"""Pins for the float64 oracle: checks against closed forms, exact rational
brute force and invariants, never against the oracle itself.

Each ``*_pin_failures(fn)`` runs every pin on a candidate implementation ``fn``
and returns the names of the pins it fails. The real oracle must fail none;
``test_oracle_mutants.py`` plants plausible mistakes in copies of the oracle and
requires each copy to fail at least one pin.
"""
from __future__ import annotations

import math
import random
from fractions import Fraction

import mpmath
import numpy as np

# --------------------------------------------------------------------------
# linear recurrence  h[t] = a[t] h[t-1] + b[t],  h[-1] = h0
# ("Selective-scan CUDA kernels", paragraph stating the recurrence)
# --------------------------------------------------------------------------


def _tree_compose(maps, rng):
    """Compose affine maps (a, b) over Fractions with a random binary tree.

    The map list is split at a random point, each half is reduced recursively
    and the halves are composed, earlier half applied first. This evaluates
    the same composition as the sequential recurrence through a different
    parenthesisation, so it is exact truth that does not retype the loop.
    """
    if len(maps) == 1:
        return maps[0]
    k = rng.randint(1, len(maps) - 1)
    a1, b1 = _tree_compose(maps[:k], rng)
    a2, b2 = _tree_compose(maps[k:], rng)
    # x -> a2*(a1*x + b1) + b2
    return (a1 * a2, a2 * b1 + b2)


def exact_linear(a, b, h0, seed=0):
    """Exact h[t] (as Fractions) via random-tree composition of the prefix maps."""
    rng = random.Random(seed)
    maps = [(Fraction(float(x)), Fraction(float(y))) for x, y in zip(a, b)]
    H0 = Fraction(float(h0))
    out = []
    for t in range(len(maps)):
        A, Bv = _tree_compose(maps[: t + 1], rng)
        out.append(A * H0 + Bv)
    return out


def _close(x, ref, rtol):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        return False
    return bool(np.all(np.abs(x - ref) <= rtol * (1.0 + np.abs(ref))))


def linear_pin_failures(scan):
    """scan(a, b, h0) -> float64 array of h. Returns names of failed pins."""
    fails = []
    rs = np.random.RandomState(7)

    # 1. exact rational brute force, random tree parenthesisations
    ok = True
    for n, lo, hi in ((1, -1, 1), (2, -1, 1), (7, -1.2, 1.2), (33, 0.5, 1.0), (64, -1, 1)):
        a = rs.uniform(lo, hi, n)
        b = rs.normal(size=n)
        h0 = rs.normal()
        truth = [float(v) for v in exact_linear(a, b, h0, seed=n)]
        if not _close(scan(a, b, h0), truth, 1e-12):
            ok = False
    if not ok:
        fails.append("fraction_bruteforce")

    # 2. constant a = c, constant b = beta: geometric series with carry-in
    ok = True
    for c, beta, h0 in ((0.5, 1.0, 0.0), (0.97, -0.3, 2.0), (-0.8, 0.7, -1.5)):
        n = 200
        t = np.arange(n) + 1
        ref = c ** t * h0 + beta * (1 - c ** t) / (1 - c)
        if not _close(scan(np.full(n, c), np.full(n, beta), h0), ref, 1e-12):
            ok = False
    if not ok:
        fails.append("geometric_closed_form")

    # 3. a == 1 with integer b: prefix sum, exact
    b = rs.randint(-1000, 1000, 500).astype(np.float64)
    ref = 17.0 + np.cumsum(b)
    if not np.array_equal(np.asarray(scan(np.ones(500), b, 17.0)), ref):
        fails.append("prefix_sum_exact")

    # 4. a == 0: h == b exactly, carry-in discarded
    b = rs.normal(size=300)
    if not np.array_equal(np.asarray(scan(np.zeros(300), b, 5.0)), b):
        fails.append("zero_a_exact")

    # 5. a in {0, 1} with integer b: segmented prefix sums, exact
    a = (rs.uniform(size=400) < 0.8).astype(np.float64)
    b = rs.randint(-50, 50, 400).astype(np.float64)
    h0 = 3.0
    seg = np.cumsum(a == 0)               # segment id; a zero starts a new segment
    ref = np.empty(400)
    for s in np.unique(seg):
        idx = np.nonzero(seg == s)[0]
        ref[idx] = np.cumsum(b[idx]) + (h0 if s == 0 else 0.0)
    if not np.array_equal(np.asarray(scan(a, b, h0)), ref):
        fails.append("segmented_sum_exact")
    return fails


# --------------------------------------------------------------------------
# S6 selective scan (POPCORNBENCH transcript FW-GLM-5-1, forward pass; reverse
# and bidirectional per "ARM-Scan", "Approach")
# --------------------------------------------------------------------------


def _rand_s6(rs, batch, L, d, N, a_lo=-2.0, a_hi=-0.1):
    u = rs.normal(size=(batch, L, d))
    delta = rs.uniform(0.05, 1.0, size=(batch, L, d))
    A = rs.uniform(a_lo, a_hi, size=(d, N))
    B = rs.normal(size=(batch, L, N))
    C = rs.normal(size=(batch, L, N))
    D = rs.normal(size=d)
    return u, delta, A, B, C, D


class _Crashed(Exception):
    pass


def _guard(fn):
    """Wrap a candidate so that any exception it raises marks the pin failed."""
    def wrapped(*args, **kwargs):
        try:
            return np.asarray(fn(*args, **kwargs), dtype=np.float64)
        except Exception as exc:  # noqa: BLE001 - a crash is a failed pin
            raise _Crashed(repr(exc)) from exc
    return wrapped


def _pin_n1_reduces_to_linear(s6, linear_scan, rs):
    """N=1, B=C=1, D=0 reduces to the linear recurrence with a = exp(delta*A),
    b = delta*u (forward), and to its mirror image for reverse."""
    batch, L, d = 2, 40, 3
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, 1)
    B = np.ones_like(B)
    C = np.ones_like(C)
    D = np.zeros_like(D)
    ok = True
    yf = s6(u, delta, A, B, C, D, "fwd")
    yr = s6(u, delta, A, B, C, D, "rev")
    for bi in range(batch):
        for di in range(d):
            a_seq = np.exp(delta[bi, :, di] * A[di, 0])
            b_seq = delta[bi, :, di] * u[bi, :, di]
            if not _close(yf[bi, :, di], linear_scan(a_seq, b_seq, 0.0), 1e-12):
                ok = False
            rev = linear_scan(a_seq[::-1], b_seq[::-1], 0.0)[::-1]
            if not _close(yr[bi, :, di], rev, 1e-12):
                ok = False
    return ok


def _pin_zero_A_exact(s6, linear_scan, rs):
    """A = 0: no decay, so h_t = sum over the visited steps of delta*B*u and
    every quantity is rational; exact Fraction evaluation of that closed form."""
    batch, L, d, N = 2, 9, 3, 4
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    A = np.zeros_like(A)
    for direction in ("fwd", "rev"):
        y = s6(u, delta, A, B, C, D, direction)
        if y.shape != u.shape:
            return False
        for bi in range(batch):
            for di in range(d):
                for t in range(L):
                    span = range(0, t + 1) if direction == "fwd" else range(t, L)
                    acc = Fraction(0)
                    for n in range(N):
                        hn = sum((Fraction(delta[bi, s, di]) * Fraction(B[bi, s, n])
                                  * Fraction(u[bi, s, di]) for s in span), Fraction(0))
                        acc += Fraction(C[bi, t, n]) * hn
                    acc += Fraction(D[di]) * Fraction(u[bi, t, di])
                    if abs(float(acc) - y[bi, t, di]) > 1e-12 * (1 + abs(float(acc))):
                        return False
    return True


def _pin_memoryless_closed_form(s6, linear_scan, rs):
    """A = -inf: dA = 0, the state keeps only the current step, so
    y_t = delta_t u_t sum_n C_tn B_tn + D u_t in both directions."""
    batch, L, d, N = 2, 15, 4, 5
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    A = np.full_like(A, -np.inf)
    ref = delta * u * np.sum(B * C, axis=-1)[:, :, None] + u * D[None, None, :]
    return _close(s6(u, delta, A, B, C, D, "fwd"), ref, 1e-13) and \
        _close(s6(u, delta, A, B, C, D, "rev"), ref, 1e-13)


def _pin_geometric_closed_form(s6, linear_scan, rs):
    """Inputs constant in t: a geometric series per (b, d, n) with ratio
    exp(delta*A[d, n]); d == N so a transposed A is a silent value error."""
    batch, L, d, N = 2, 30, 3, 3
    ub = rs.normal(size=(batch, 1, d))
    db = rs.uniform(0.1, 0.9, size=(batch, 1, d))
    Bb = rs.normal(size=(batch, 1, N))
    Cb = rs.normal(size=(batch, 1, N))
    A = -np.array([[0.3, 1.1, 2.0], [0.7, 0.2, 1.6], [1.3, 0.5, 0.9]])
    D = rs.normal(size=d)
    u = np.repeat(ub, L, axis=1)
    delta = np.repeat(db, L, axis=1)
    B = np.repeat(Bb, L, axis=1)
    C = np.repeat(Cb, L, axis=1)
    for direction in ("fwd", "rev"):
        y = s6(u, delta, A, B, C, D, direction)
        ref = np.zeros((batch, L, d))
        for bi in range(batch):
            for di in range(d):
                for t in range(L):
                    k = t + 1 if direction == "fwd" else L - t
                    acc = 0.0
                    for n in range(N):
                        r = math.exp(db[bi, 0, di] * A[di, n])
                        hn = db[bi, 0, di] * ub[bi, 0, di] * Bb[bi, 0, n] * (1 - r ** k) / (1 - r)
                        acc += Cb[bi, 0, n] * hn
                    ref[bi, t, di] = acc + D[di] * ub[bi, 0, di]
        if not _close(y, ref, 1e-11):
            return False
    return True


def _pin_zero_B_skip_only(s6, linear_scan, rs):
    """B = 0: the state stays zero, y = D*u exactly (twice for bidir)."""
    batch, L, d, N = 2, 20, 3, 4
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    B = np.zeros_like(B)
    return np.array_equal(s6(u, delta, A, B, C, D, "fwd"), u * D) and \
        np.array_equal(s6(u, delta, A, B, C, D, "rev"), u * D) and \
        np.array_equal(s6(u, delta, A, B, C, D, "bidir"), 2 * (u * D))


def _pin_bidir_identity(s6, linear_scan, rs):
    """bidir == fwd + rev, and rev == flip_L . fwd . flip_L."""
    batch, L, d, N = 2, 25, 3, 4
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    yf = s6(u, delta, A, B, C, D, "fwd")
    yr = s6(u, delta, A, B, C, D, "rev")
    yb = s6(u, delta, A, B, C, D, "bidir")
    fl = lambda x: x[:, ::-1]  # noqa: E731
    yflip = fl(s6(fl(u), fl(delta), A, fl(B), fl(C), D, "fwd"))
    return _close(yb, yf + yr, 1e-13) and _close(yr, yflip, 1e-13)


def _pin_causality(s6, linear_scan, rs):
    """Changing inputs at t >= t0 leaves forward outputs before t0 untouched
    (and changes later ones); changing inputs at t <= t0 leaves reverse outputs
    after t0 untouched."""
    batch, L, d, N = 2, 25, 3, 4
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    yf = s6(u, delta, A, B, C, D, "fwd")
    yr = s6(u, delta, A, B, C, D, "rev")
    t0 = 11

    def bump(sl):
        u2, d2, B2, C2 = u.copy(), delta.copy(), B.copy(), C.copy()
        u2[:, sl] += 1.0
        d2[:, sl] *= 1.5
        B2[:, sl] -= 0.5
        C2[:, sl] += 0.25
        return u2, d2, B2, C2

    u2, d2, B2, C2 = bump(slice(t0, None))
    yf2 = s6(u2, d2, A, B2, C2, D, "fwd")
    u3, d3, B3, C3 = bump(slice(0, t0 + 1))
    yr2 = s6(u3, d3, A, B3, C3, D, "rev")
    return (np.array_equal(yf2[:, :t0], yf[:, :t0]) and
            np.array_equal(yr2[:, t0 + 1:], yr[:, t0 + 1:]) and
            not np.allclose(yf2[:, t0:], yf[:, t0:]))


def _pin_permutation_equivariance(s6, linear_scan, rs):
    """Permuting channels (u, delta, A rows, D) or batch entries permutes y the
    same way; d != N so a d/n mix-up shows."""
    batch, L, d, N = 3, 12, 5, 4
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    yb = s6(u, delta, A, B, C, D, "bidir")
    perm_d = np.array([3, 0, 4, 1, 2])
    perm_b = np.array([2, 0, 1])
    yp = s6(u[perm_b][:, :, perm_d], delta[perm_b][:, :, perm_d], A[perm_d],
            B[perm_b], C[perm_b], D[perm_d], "bidir")
    return _close(yp, yb[perm_b][:, :, perm_d], 1e-13)


def _pin_linearity_in_u(s6, linear_scan, rs):
    """With delta, A, B, C fixed, y is linear in u."""
    batch, L, d, N = 2, 16, 3, 4
    u, delta, A, B, C, D = _rand_s6(rs, batch, L, d, N)
    up = rs.normal(size=u.shape)
    lhs = s6(2 * u + 0.5 * up, delta, A, B, C, D, "bidir")
    rhs = 2 * s6(u, delta, A, B, C, D, "bidir") + 0.5 * s6(up, delta, A, B, C, D, "bidir")
    return _close(lhs, rhs, 1e-12)


_S6_PINS = [
    ("n1_reduces_to_linear", _pin_n1_reduces_to_linear),
    ("zero_A_exact", _pin_zero_A_exact),
    ("memoryless_closed_form", _pin_memoryless_closed_form),
    ("geometric_closed_form", _pin_geometric_closed_form),
    ("zero_B_skip_only", _pin_zero_B_skip_only),
    ("bidir_identity", _pin_bidir_identity),
    ("causality", _pin_causality),
    ("permutation_equivariance", _pin_permutation_equivariance),
    ("linearity_in_u", _pin_linearity_in_u),
]


def s6_pin_failures(s6, linear_scan):
    """s6(u, delta, A, B, C, D, direction) -> y (float64). ``linear_scan`` is the
    (already pinned) linear oracle used by the N=1 reduction pin. A candidate
    that raises inside a pin fails that pin. Returns names of failed pins."""
    fails = []
    s6 = _guard(s6)
    for i, (name, pin) in enumerate(_S6_PINS):
        rs = np.random.RandomState(100 + i)
        try:
            ok = pin(s6, linear_scan, rs)
        except _Crashed:
            ok = False
        if not ok:
            fails.append(name)
    return fails


# ---------------------------------------------------------------- softplus ---
#
# softplus(x) = log(1 + exp(x)), which the POPCORNBENCH transcript's model
# applies to the delta projection (bias included) before the scan.

def softplus_pin_failures(softplus):
    """softplus(x) -> float64 array. Returns names of failed pins."""
    fails = []
    sp = _guard(softplus)
    rs = np.random.RandomState(11)
    x = np.concatenate([rs.normal(scale=4.0, size=200), [-60.0, -30.0, -1e-9, 1e-9, 30.0]])
    checks = {
        # log 2 at zero
        "value_at_zero": lambda: abs(float(sp(np.array([0.0]))[0]) - math.log(2.0)) <= 1e-15,
        # log(1 + e^x) - log(1 + e^-x) = log(e^x) = x
        "odd_part_is_x": lambda: _close(sp(x) - sp(-x), x, 1e-13),
        # softplus(x) = e^x - e^2x / 2 + ... for x << 0: relatively within e^x + rounding
        "small_tail": lambda: bool(np.all(
            np.abs(sp(np.array([-30.0, -40.0, -700.0])) / np.exp([-30.0, -40.0, -700.0]) - 1.0)
            <= 1e-15 + np.exp([-30.0, -40.0, -700.0]))),
        # softplus(x) = x + e^-x - ... for x >> 0, and no overflow
        "large_tail": lambda: _close(sp(np.array([50.0, 1000.0])), [50.0, 1000.0], 1e-15),
        # against 50-digit log(1 + exp(x)) at a few points
        "mpmath_values": lambda: _softplus_vs_mpmath(sp),
    }
    for name, check in checks.items():
        try:
            ok = check()
        except _Crashed:
            ok = False
        if not ok:
            fails.append(name)
    return fails


def _softplus_vs_mpmath(sp):
    mpmath.mp.dps = 50
    pts = [-20.0, -3.5, -0.25, 0.0, 0.7, 2.0, 9.0, 35.0]
    got = sp(np.array(pts))
    ref = [float(mpmath.log(1 + mpmath.exp(mpmath.mpf(p)))) for p in pts]
    return _close(got, ref, 1e-14)
