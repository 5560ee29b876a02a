"""The C float64 twin of the oracle against the same pins and the Python oracle."""
import numpy as np
import pytest

import oracle
from oracle import native
from pins import linear_pin_failures, s6_pin_failures


def c_s6(u, delta, A, B, C, D, direction):
    return native.selective_scan(u, delta, A, B, C, D, direction, nthreads=2)[0]


def test_c_linear_passes_pins():
    assert linear_pin_failures(native.linear_scan) == []


def test_c_s6_passes_pins():
    assert s6_pin_failures(c_s6, native.linear_scan) == []


@pytest.mark.parametrize("direction", ["fwd", "rev", "bidir"])
def test_c_twin_matches_python_oracle(direction):
    rs = np.random.RandomState(4)
    batch, L, d, N = 3, 50, 5, 16
    u = rs.normal(size=(batch, L, d))
    delta = rs.uniform(0.01, 2.0, size=(batch, L, d))
    A = -rs.uniform(0.5, 16, size=(d, N))
    B = rs.normal(size=(batch, L, N))
    C = rs.normal(size=(batch, L, N))
    D = rs.normal(size=d)
    ref = oracle.selective_scan(u, delta, A, B, C, D, direction)
    got = c_s6(u, delta, A, B, C, D, direction)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_c_channel_range_only_writes_its_channels():
    rs = np.random.RandomState(8)
    batch, L, d, N = 2, 7, 3, 4
    u = rs.normal(size=(batch, L, d))
    delta = rs.uniform(0.1, 1.0, size=(batch, L, d))
    A = -rs.uniform(0.5, 2, size=(d, N))
    B = rs.normal(size=(batch, L, N))
    C = rs.normal(size=(batch, L, N))
    D = rs.normal(size=d)
    full = c_s6(u, delta, A, B, C, D, "fwd")
    part, _ = native.selective_scan(u, delta, A, B, C, D, "fwd", ch_begin=2, ch_end=4)
    flat_full = full.transpose(0, 2, 1).reshape(batch * d, L)
    flat_part = part.transpose(0, 2, 1).reshape(batch * d, L)
    assert np.array_equal(flat_part[2:4], flat_full[2:4])
    assert np.isnan(flat_part[:2]).all() and np.isnan(flat_part[4:]).all()


def test_c_linear_matches_python_oracle_long():
    rs = np.random.RandomState(2)
    a = rs.uniform(0.5, 1.0, 100000)
    b = rs.normal(size=100000)
    assert np.array_equal(native.linear_scan(a, b, 0.3), oracle.linear_scan(a, b, 0.3))
