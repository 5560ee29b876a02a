"""Non-finite inputs: every linear scan (single-pass, three-pass, Hillis-Steele
and batched) against the float64 oracle element by element, with NaN and
+-inf positions (and signs) compared exactly.

The sequential loop h = a*h + b never multiplies multipliers together; the
scans do, and a long product of multipliers below 1 underflows in fp32. The
cases plant inf/NaN in b, h0 and a, exact zeros after an infinite state, and
place them at the first element, inside rows, at row, wave and tile ends, in
later superblocks and in the ragged last tile, with a ~ U(0.5, 1) so that
products over a tile underflow.
"""
import numpy as np
import pytest
import torch

import mamba_s6_selective_amd as ssm
from gpu_util import assert_same_nonfinite, need_gpu, say
from mamba_s6_selective_amd.workloads import linear_inputs
from oracle import native

pytestmark = pytest.mark.gpu
TOL = 1e-4
INF, NAN = float("inf"), float("nan")
N = 300 * 8192 + 77          # 301 tiles of the single-pass and three-pass scans: level-1 windows
POS = [0, 5, 1023, 8191, 64 * 8192 + 300, N - 1]   # first, in a row, wave end, tile end, later, last

# name -> list of (array, offset into POS or absolute position, value), h0
CASES = {
    "b+inf": ([("b", 0, INF)], 0.0),
    "b-inf": ([("b", 0, -INF)], 0.0),
    "bnan": ([("b", 0, NAN)], 0.0),
    "b+inf then b-inf": ([("b", 0, INF), ("b", 7777, -INF)], 0.0),
    "b+inf then a=0": ([("b", 0, INF), ("a", 9000, 0.0)], 0.0),
    "a+inf": ([("a", 0, INF)], 0.5),
    "a-inf": ([("a", 0, -INF)], 0.5),
    "anan": ([("a", 0, NAN)], 0.5),
    "a=0 then a+inf": ([("a", 0, 0.0), ("a", 3000, INF)], 0.5),
    "two a+inf": ([("a", 0, INF), ("a", 20000, -INF)], 0.5),
}


def planted(case, p, n=N, seed=4242):
    a, b = linear_inputs(n, seed=seed, a_lo=0.5, a_hi=1.0)
    plants, h0 = CASES[case]
    for arr, delta, v in plants:
        i = min(p + delta, n - 1)
        (a if arr == "a" else b)[i] = v
    return a, b, h0


SCANS = {"single": ssm.linear_scan, "3pass": ssm.linear_scan_3pass, "hs": ssm.linear_scan_hs}


@pytest.mark.parametrize("scan", sorted(SCANS))
@pytest.mark.parametrize("p", POS)
@pytest.mark.parametrize("case", sorted(CASES))
def test_nonfinite_linear(case, p, scan):
    say(f"nonfinite {scan}: {case} at {p}")
    dev = need_gpu()
    a, b, h0 = planted(case, p)
    h = SCANS[scan](a.to(dev), b.to(dev), h0).cpu().numpy()
    ref = native.linear_scan(a.numpy(), b.numpy(), h0)
    assert_same_nonfinite(h, ref, TOL, f"{scan} {case}@{p}")


@pytest.mark.parametrize("scan", sorted(SCANS))
@pytest.mark.parametrize("h0", [INF, -INF, NAN])
def test_nonfinite_h0(scan, h0):
    say(f"nonfinite {scan}: h0 = {h0}")
    dev = need_gpu()
    a, b = linear_inputs(70 * 8192 + 5, seed=11, a_lo=0.5, a_hi=1.0)
    h = SCANS[scan](a.to(dev), b.to(dev), h0).cpu().numpy()
    ref = native.linear_scan(a.numpy(), b.numpy(), h0)
    assert_same_nonfinite(h, ref, TOL, f"{scan} h0={h0}")


@pytest.mark.parametrize("scan", sorted(SCANS))
def test_nonfinite_small_multipliers_everywhere(scan):
    """a ~ U(0, 0.01): products underflow within a few elements everywhere;
    an inf in b must stay inf through them (and later NaN from an exact 0)."""
    dev = need_gpu()
    n = 40 * 8192 + 3
    a, b = linear_inputs(n, seed=12, a_lo=0.0, a_hi=0.01)
    b[1234] = INF
    b[5 * 8192 + 17] = -INF
    a[20 * 8192] = 0.0
    b[30 * 8192 + 1] = NAN
    h = SCANS[scan](a.to(dev), b.to(dev), 0.25).cpu().numpy()
    ref = native.linear_scan(a.numpy(), b.numpy(), 0.25)
    assert_same_nonfinite(h, ref, TOL, f"{scan} small a")


@pytest.mark.parametrize("scan", sorted(SCANS))
@pytest.mark.parametrize("n", [1, 3, 4, 5, 257, 8193])
def test_nonfinite_tiny_sizes(scan, n):
    dev = need_gpu()
    for case in ("b+inf", "a-inf", "bnan"):
        a, b, h0 = planted(case, n // 2, n=n, seed=n)
        h = SCANS[scan](a.to(dev), b.to(dev), h0).cpu().numpy()
        ref = native.linear_scan(a.numpy(), b.numpy(), h0)
        assert_same_nonfinite(h, ref, TOL, f"{scan} n={n} {case}")


# batched: shapes with long sequences (several tiles each), many short ones
# per tile, and length-1 sequences
BATCHED = [(24, 40000), (500, 1000), (3000, 3), (9, 8448 * 3 + 1)]


@pytest.mark.parametrize("shape", BATCHED, ids=[f"{s[0]}x{s[1]}" for s in BATCHED])
def test_nonfinite_batched_all_sequences(shape):
    """inf / NaN in b, h0 and a inside some sequences, at their first and
    last elements and in between; every sequence, those holding the values
    included, against the oracle run on that sequence alone, and h_last."""
    nseq, length = shape
    say(f"nonfinite batched {nseq} x {length}")
    dev = need_gpu()
    g = torch.Generator().manual_seed(nseq + length)
    a = 0.5 + 0.5 * torch.rand(nseq, length, generator=g)
    b = torch.randn(nseq, length, generator=g)
    h0 = torch.randn(nseq, generator=g)
    mid = length // 2
    b[1, mid] = INF                        # inf inside a sequence
    h0[2] = INF                            # an infinite start
    h0[3] = NAN
    b[4, 0] = -INF                         # at a sequence's first element
    b[5, length - 1] = NAN                 # at its last: the next one is unaffected
    a[6, mid] = INF                        # an infinite multiplier
    b[7, 0] = INF
    if length > 1:
        a[7, length - 1] = 0.0             # then an exact zero: NaN
        a[0, length - 1] = -INF            # at a last element, sequence 0
    if nseq > 100:
        b[100, mid] = -INF
        a[101, 0] = INF                    # infinite multiplier at a first element
    h, last = ssm.linear_scan_batched(a.to(dev), b.to(dev), h0.to(dev))
    h, last = h.cpu().numpy(), last.cpu().numpy()
    ref = np.stack([native.linear_scan(a[k].numpy(), b[k].numpy(), float(h0[k]))
                    for k in range(nseq)])
    assert_same_nonfinite(h, ref, TOL, f"batched {nseq}x{length}")
    assert_same_nonfinite(last, ref[:, -1], TOL, "h_last")
    assert np.array_equal(last, h[:, -1], equal_nan=True)  # the same values, bit for bit


# ---- S6: non-finite inputs through the chunk, carry and fix passes ---------

import oracle  # noqa: E402
from mamba_s6_selective_amd.workloads import s6_inputs  # noqa: E402

S6_CASES = {
    # name -> list of (tensor, index, value); indices are (b, t, d) or (b, t, n)
    "u+inf": [("u", (0, 700, 5), INF)],
    "u-inf": [("u", (1, 1500, 9), -INF)],
    "unan": [("u", (0, 300, 3), NAN)],
    "u+inf then u-inf": [("u", (0, 700, 5), INF), ("u", (0, 1900, 5), -INF)],
    # a huge delta: that step's exponential flushes in fp32 (the float64 value
    # is tiny, not zero) right after an infinite state
    "u+inf then huge delta": [("u", (0, 850, 7), INF), ("delta", (0, 900, 7), 200.0)],
    "delta+inf": [("delta", (1, 1234, 2), INF)],
    "B+inf": [("B", (0, 1000, 0), INF)],
    "C+inf": [("C", (1, 2000, 0), -INF)],
    "C=0 on an infinite state": [("u", (0, 700, 5), INF), ("C", (0, 1200, 0), 0.0)],
}


def s6_planted(case, N, seed=31):
    inp = s6_inputs(2, 3000, 64, N, seed=seed, dtype="f32")
    if N == 1:  # the first-order recurrence per channel: a = exp(delta A), b = delta u
        inp.B = torch.ones_like(inp.B)
        inp.C = torch.ones_like(inp.C)
        inp.D = torch.zeros_like(inp.D)
    for name, idx, v in S6_CASES[case]:
        getattr(inp, name)[idx] = v
    return inp


@pytest.mark.parametrize("chunk", ["256", None])
@pytest.mark.parametrize("N", [1, 16])
@pytest.mark.parametrize("case", sorted(S6_CASES))
def test_nonfinite_s6(case, N, chunk, monkeypatch):
    """Every output against the float64 oracle, NaN and +-inf positions and
    signs included, forward, reverse and bidirectional, with chunks of 256
    steps (carries cross 11 chunk boundaries) and with the planner's."""
    say(f"nonfinite s6 {case} N={N} chunk={chunk}")
    if chunk:
        monkeypatch.setenv("SSMSCAN_S6_CHUNK", chunk)
    else:
        monkeypatch.delenv("SSMSCAN_S6_CHUNK", raising=False)
    dev = need_gpu()
    inp = s6_planted(case, N)
    t = [x.to(dev) for x in (inp.u, inp.delta, inp.A, inp.B, inp.C, inp.D)]
    for direction in ("fwd", "rev", "bidir"):
        y = ssm.selective_scan_fwd(*t, direction=direction).cpu().numpy()
        with np.errstate(all="ignore"):
            ref = oracle.selective_scan(*inp.as_f64(), direction=direction)
        assert_same_nonfinite(y, ref, TOL, f"s6 {case} N={N} {direction}")


@pytest.mark.parametrize("chunk", ["256", None])
@pytest.mark.parametrize("N", [1, 16])
def test_nonfinite_s6_flush_in_reverse_only(N, chunk, monkeypatch):
    """L = 3003: the last chunk ends in a tail of 3 steps that the forward
    sweep takes one step at a time, while the reverse sweep takes them in
    its first full block of 8. u = +inf at the last step and a huge delta one
    step before it meet only in the reverse recurrence (an infinite state
    times an exponential that flushes in fp32), so in the bidirectional call
    only the reverse sweep has to be evaluated again, after the forward
    output is formed again. Every output against the float64 oracle."""
    say(f"nonfinite s6 flush in reverse only N={N} chunk={chunk}")
    if chunk:
        monkeypatch.setenv("SSMSCAN_S6_CHUNK", chunk)
    else:
        monkeypatch.delenv("SSMSCAN_S6_CHUNK", raising=False)
    dev = need_gpu()
    inp = s6_inputs(2, 3003, 64, N, seed=37, dtype="f32")
    if N == 1:
        inp.B = torch.ones_like(inp.B)
        inp.C = torch.ones_like(inp.C)
        inp.D = torch.zeros_like(inp.D)
    inp.u[0, 3002, 7] = INF
    inp.delta[0, 3001, 7] = 200.0
    t = [x.to(dev) for x in (inp.u, inp.delta, inp.A, inp.B, inp.C, inp.D)]
    for direction in ("fwd", "rev", "bidir"):
        y = ssm.selective_scan_fwd(*t, direction=direction).cpu().numpy()
        with np.errstate(all="ignore"):
            ref = oracle.selective_scan(*inp.as_f64(), direction=direction)
        assert_same_nonfinite(y, ref, TOL, f"s6 reverse-only flush N={N} {direction}")
