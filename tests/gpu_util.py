"""Helpers for the GPU parity tests (comparison against the float64 oracle)."""
import sys

import numpy as np
import torch

import mamba_s6_selective_amd as ssm


def need_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    ssm.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def max_scaled_err(got, ref):
    """max |got - ref| / (1 + |ref|) over all elements (NaN-aware: positions
    must agree)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn), "NaN positions differ"
    m = ~rn
    if not m.any():
        return 0.0
    return float(np.max(np.abs(got[m] - ref[m]) / (1.0 + np.abs(ref[m]))))


def assert_close(got, ref, tol, what=""):
    err = max_scaled_err(got, ref)
    say(f"  {what}: max |err|/(1+|ref|) = {err:.3e} (tol {tol:g})")
    assert err <= tol, f"{what}: {err} > {tol}"


def assert_same_nonfinite(got, ref, tol, what=""):
    """Element by element against the oracle with non-finite values included:
    NaN where the oracle has NaN, +inf / -inf where it has +inf / -inf (sign
    included), and the finite values within tol * (1 + |ref|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    for name, fn in (("NaN", np.isnan), ("+inf", np.isposinf), ("-inf", np.isneginf)):
        g, r = fn(got), fn(ref)
        if not np.array_equal(g, r):
            bad = np.flatnonzero(g != r)
            raise AssertionError(
                f"{what}: {name} positions differ at {bad.size} elements, first "
                f"{bad[:5].tolist()} (got {got.ravel()[bad[:5]].tolist()}, "
                f"oracle {ref.ravel()[bad[:5]].tolist()})")
    m = np.isfinite(ref)
    err = float(np.max(np.abs(got[m] - ref[m]) / (1.0 + np.abs(ref[m])))) if m.any() else 0.0
    say(f"  {what}: {int((~m).sum())} non-finite matched, finite max err {err:.3e}")
    assert err <= tol, f"{what}: {err} > {tol}"
