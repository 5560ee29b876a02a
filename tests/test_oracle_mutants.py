"""Mutation tests: copies of the oracle with one planted mistake each must fail
at least one pin. This is what shows the pins would catch a plausible error in
the oracle (a swapped operand, a dropped term, a wrong sign or index), in the
spirit of the deliberately broken index-arithmetic mirrors described in
"Selective-scan CUDA kernels" (the paragraph on correctness and determinism).
All mistakes are planted here, on the CPU, never in GPU code.
"""
import numpy as np
import pytest

import oracle
from pins import linear_pin_failures, s6_pin_failures

# ---------------------------------------------------------------- linear ---


def _pair_scan_with(combine, fold_right=False):
    def scan(a, b, h0):
        acc, out = None, []
        for at, bt in zip(map(float, a), map(float, b)):
            m = (at, bt)
            if acc is None:
                acc = m
            elif fold_right:
                acc = combine(m, acc)          # later map composed first
            else:
                acc = combine(acc, m)
            out.append(oracle.apply_affine(acc, float(h0)))
        return np.array(out)
    return scan


def swapped_combine(p, q):
    a1, b1 = p
    a2, b2 = q
    return (a1 * a2, a1 * b2 + b1)


def _loop_mutant(kind):
    def scan(a, b, h0):
        a = np.asarray(a, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        h, out = float(h0), []
        if kind == "ignore_h0":
            h = 0.0
        for t in range(len(a)):
            if kind == "b_prev":
                h = a[t] * h + (b[t - 1] if t > 0 else 0.0)
            elif kind == "a_prev":
                h = (a[t - 1] if t > 0 else 1.0) * h + b[t]
            elif kind == "scale_b_too":
                h = a[t] * (h + b[t])
            elif kind == "exclusive":
                out.append(h)
                h = a[t] * h + b[t]
                continue
            else:
                h = a[t] * h + b[t]
            out.append(h)
        return np.array(out)
    return scan


LINEAR_MUTANTS = {
    "swapped_combine": _pair_scan_with(swapped_combine),
    "right_fold": _pair_scan_with(oracle.affine_combine, fold_right=True),
    "ignore_h0": _loop_mutant("ignore_h0"),
    "b_prev": _loop_mutant("b_prev"),
    "a_prev": _loop_mutant("a_prev"),
    "scale_b_too": _loop_mutant("scale_b_too"),
    "exclusive": _loop_mutant("exclusive"),
}


@pytest.mark.parametrize("name", sorted(LINEAR_MUTANTS))
def test_linear_mutant_is_caught(name):
    assert linear_pin_failures(LINEAR_MUTANTS[name]) != [], name


def test_swapped_combine_caught_by_bruteforce_specifically():
    # constant a cannot tell the two composition orders apart; random a can
    fails = linear_pin_failures(LINEAR_MUTANTS["swapped_combine"])
    assert "fraction_bruteforce" in fails
    assert "geometric_closed_form" not in fails


# -------------------------------------------------------------------- S6 ---


def _s6_mutant(kind):
    """A copy of oracle.s6's loop with one planted mistake."""

    def one(u, delta, A, B, C, D, reverse):
        batch, L, d = u.shape
        N = A.shape[1]
        h = np.zeros((batch, d, N))
        y = np.empty((batch, L, d))
        steps = list(range(L - 1, -1, -1)) if reverse else list(range(L))
        AA = A.T if kind == "A_transposed" else A
        for t in steps:
            dt = delta[:, t, :]
            x = u[:, t, :]
            if kind == "rev_shifted_discretization" and reverse:
                tt = min(t + 1, L - 1)
                dt_a = delta[:, tt, :]
            else:
                dt_a = dt
            if kind == "sign_A":
                dA = np.exp(-dt_a[:, :, None] * AA[None])
            elif kind == "dA_no_delta":
                dA = np.exp(AA[None] + 0 * dt_a[:, :, None])
            elif kind == "u_in_dA":
                dA = np.exp(x[:, :, None] * AA[None])
            else:
                dA = np.exp(dt_a[:, :, None] * AA[None])
            Bt = C[:, t, None, :] if kind == "B_C_swapped" else B[:, t, None, :]
            dB = Bt if kind == "dB_no_delta" else dt[:, :, None] * Bt
            x_db = x[:, :, None] * dB
            h_prev = h
            h = dA * h + x_db
            hy = h_prev if kind == "y_before_update" else h
            if kind == "C_prev":
                Ct = C[:, t - 1, None, :]
            elif kind == "B_C_swapped":
                Ct = B[:, t, None, :]
            else:
                Ct = C[:, t, None, :]
            skip = 0.0 if kind == "drop_D" else x * D[None, :]
            y[:, t, :] = np.sum(hy * Ct, axis=-1) + skip
        return y

    def s6(u, delta, A, B, C, D, direction="fwd"):
        u, delta, A, B, C, D = (np.asarray(v, dtype=np.float64) for v in (u, delta, A, B, C, D))
        if direction == "fwd":
            return one(u, delta, A, B, C, D, False)
        if direction == "rev":
            return one(u, delta, A, B, C, D, True)
        y = one(u, delta, A, B, C, D, False) + one(u, delta, A, B, C, D, True)
        if kind == "bidir_D_once":
            y = y - u * D[None, None, :]
        return y
    return s6


S6_MUTANTS = ["y_before_update", "C_prev", "drop_D", "sign_A", "A_transposed",
              "dB_no_delta", "dA_no_delta", "u_in_dA", "B_C_swapped",
              "rev_shifted_discretization", "bidir_D_once"]


def test_unmutated_copy_passes():
    assert s6_pin_failures(_s6_mutant("none"), oracle.linear_scan) == []


@pytest.mark.parametrize("name", S6_MUTANTS)
def test_s6_mutant_is_caught(name):
    # some mutants (a flipped sign of A, u in the exponent) overflow; that is
    # part of how they fail
    with np.errstate(over="ignore", invalid="ignore"):
        failures = s6_pin_failures(_s6_mutant(name), oracle.linear_scan)
    assert failures != [], name


# -------------------------------------------------------------- softplus ---

SOFTPLUS_MUTANTS = {
    "naive_overflow": lambda x: np.log(1.0 + np.exp(np.asarray(x, dtype=np.float64))),
    "missing_exp": lambda x: np.log1p(np.abs(np.asarray(x, dtype=np.float64))),
    "wrong_sign": lambda x: np.logaddexp(0.0, -np.asarray(x, dtype=np.float64)),
    "relu_only": lambda x: np.maximum(np.asarray(x, dtype=np.float64), 0.0),
    "log2_base": lambda x: np.logaddexp2(0.0, np.asarray(x, dtype=np.float64)),
}


@pytest.mark.parametrize("name", sorted(SOFTPLUS_MUTANTS))
def test_softplus_mutant_is_caught(name):
    from pins import softplus_pin_failures
    with np.errstate(all="ignore"):
        assert softplus_pin_failures(SOFTPLUS_MUTANTS[name]) != [], name
