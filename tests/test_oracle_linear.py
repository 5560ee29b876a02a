"""The float64 linear-recurrence oracle against its pins (CPU only)."""
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from pins import exact_linear, linear_pin_failures, _tree_compose


def test_linear_oracle_passes_pins():
    assert linear_pin_failures(oracle.linear_scan) == []


def pair_scan(a, b, h0):
    """The recurrence evaluated as an inclusive prefix over affine pairs."""
    return np.array([oracle.apply_affine(p, float(h0))
                     for p in oracle.affine_prefix(list(map(float, a)), list(map(float, b)))])


def test_affine_prefix_passes_pins():
    assert linear_pin_failures(pair_scan) == []


def test_affine_combine_is_associative_not_commutative():
    rng = random.Random(3)
    for _ in range(50):
        m = [(Fraction(rng.randint(-9, 9), rng.randint(1, 9)),
              Fraction(rng.randint(-9, 9), rng.randint(1, 9))) for _ in range(3)]
        left = oracle.affine_combine(oracle.affine_combine(m[0], m[1]), m[2])
        right = oracle.affine_combine(m[0], oracle.affine_combine(m[1], m[2]))
        assert left == right
    p, q = (Fraction(2), Fraction(3)), (Fraction(5), Fraction(7))
    assert oracle.affine_combine(p, q) != oracle.affine_combine(q, p)
    # q(p(x)) with p: x -> 2x+3, q: x -> 5x+7  =>  10x + 22
    assert oracle.affine_combine(p, q) == (10, 22)


def test_tree_truth_matches_plain_rational_definition():
    """The brute-force truth used by the pins equals the recurrence written over
    Fractions (checks the checker on tiny inputs)."""
    rs = np.random.RandomState(5)
    a = rs.uniform(-1, 1, 12)
    b = rs.normal(size=12)
    h = Fraction(0.25)
    want = []
    for x, y in zip(a, b):
        h = Fraction(x) * h + Fraction(y)
        want.append(h)
    assert exact_linear(a, b, 0.25, seed=9) == want


def test_empty_and_single():
    assert oracle.linear_scan([], [], 1.0).shape == (0,)
    assert oracle.linear_scan([0.5], [2.0], 4.0).tolist() == [4.0]


def test_ieee_propagation():
    h = oracle.linear_scan([1.0, 1.0, 0.0, 1.0], [np.nan, 1.0, 2.0, 1.0], 0.0)
    assert np.isnan(h[0]) and np.isnan(h[1])
    # 0 * NaN is NaN under IEEE rules: the NaN survives a zero coefficient
    assert np.isnan(h[2]) and np.isnan(h[3])
