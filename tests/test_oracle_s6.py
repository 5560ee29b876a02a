"""The float64 S6 oracle against its pins (CPU only)."""
import mpmath
import numpy as np

import oracle
from pins import s6_pin_failures


def test_s6_oracle_passes_pins():
    assert s6_pin_failures(oracle.selective_scan, oracle.linear_scan) == []


def test_s6_high_precision_bruteforce():
    """50-digit evaluation of the forward/reverse recurrence on a tiny shape."""
    mpmath.mp.dps = 50
    rs = np.random.RandomState(21)
    batch, L, d, N = 1, 6, 2, 3
    u = rs.normal(size=(batch, L, d))
    delta = rs.uniform(0.05, 1.5, size=(batch, L, d))
    A = -rs.uniform(0.1, 3.0, size=(d, N))
    B = rs.normal(size=(batch, L, N))
    C = rs.normal(size=(batch, L, N))
    D = rs.normal(size=d)
    mp = mpmath.mpf
    for direction in ("fwd", "rev", "bidir"):
        y = oracle.selective_scan(u, delta, A, B, C, D, direction)
        for di in range(d):
            ref = [mp(0)] * L
            for rev in ((False, True) if direction == "bidir" else (direction == "rev",)):
                h = [mp(0)] * N
                for t in (range(L - 1, -1, -1) if rev else range(L)):
                    dt, x = mp(delta[0, t, di]), mp(u[0, t, di])
                    for n in range(N):
                        h[n] = mpmath.exp(dt * mp(A[di, n])) * h[n] + dt * mp(B[0, t, n]) * x
                    ref[t] += sum(h[n] * mp(C[0, t, n]) for n in range(N)) + x * mp(D[di])
            for t in range(L):
                assert abs(float(ref[t]) - y[0, t, di]) <= 1e-13 * (1 + abs(float(ref[t])))


def test_s6_shape_checks():
    rs = np.random.RandomState(0)
    u = rs.normal(size=(1, 4, 3))
    A = -np.ones((3, 2))
    B = rs.normal(size=(1, 4, 2))
    try:
        oracle.selective_scan(u, u, A.T, B, B, np.ones(3))
    except ValueError:
        pass
    else:
        raise AssertionError("transposed A must be rejected")


def test_softplus_passes_pins():
    from pins import softplus_pin_failures
    assert softplus_pin_failures(oracle.softplus) == []


def test_s6_delta_softplus_bruteforce():
    """50-digit evaluation with delta_eff = log(1 + exp(delta + bias[d])),
    bias added before the softplus, against the oracle's fused option."""
    mpmath.mp.dps = 50
    rs = np.random.RandomState(23)
    batch, L, d, N = 1, 5, 3, 2
    u = rs.normal(size=(batch, L, d))
    delta = rs.normal(-1.0, 1.5, size=(batch, L, d))
    bias = rs.normal(size=d)
    A = -rs.uniform(0.1, 3.0, size=(d, N))
    B = rs.normal(size=(batch, L, N))
    C = rs.normal(size=(batch, L, N))
    D = rs.normal(size=d)
    mp = mpmath.mpf
    y = oracle.selective_scan(u, delta, A, B, C, D, "fwd", delta_bias=bias, delta_softplus=True)
    for di in range(d):
        h = [mp(0)] * N
        for t in range(L):
            dt = mpmath.log(1 + mpmath.exp(mp(delta[0, t, di]) + mp(bias[di])))
            x = mp(u[0, t, di])
            for n in range(N):
                h[n] = mpmath.exp(dt * mp(A[di, n])) * h[n] + dt * mp(B[0, t, n]) * x
            ref = sum(h[n] * mp(C[0, t, n]) for n in range(N)) + x * mp(D[di])
            assert abs(float(ref) - y[0, t, di]) <= 1e-13 * (1 + abs(float(ref)))


def test_s6_delta_bias_needs_softplus():
    rs = np.random.RandomState(0)
    u = rs.normal(size=(1, 4, 3))
    B = rs.normal(size=(1, 4, 2))
    try:
        oracle.selective_scan(u, u, -np.ones((3, 2)), B, B, np.ones(3), delta_bias=np.ones(3))
    except ValueError:
        pass
    else:
        raise AssertionError("delta_bias without delta_softplus must be rejected")
