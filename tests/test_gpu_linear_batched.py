"""GPU parity of the batched linear scan (independent sequences with their own
carry-in and carry-out) against the float64 oracle run sequence by sequence.

Bar: max |err| <= 1e-4 * (1 + |ref|) for fp32; h_last equal to the last
column of h bit for bit; bitwise identical from run to run.
"""
import numpy as np
import pytest
import torch

import mamba_s6_selective_amd as ssm
import oracle
from gpu_util import assert_close, assert_same_nonfinite, need_gpu, say
from oracle import native

pytestmark = pytest.mark.gpu
TOL = 1e-4


def inputs(nseq, length, seed, lo=0.5, hi=1.0):
    g = torch.Generator().manual_seed(seed)
    a = lo + (hi - lo) * torch.rand(nseq, length, generator=g)
    b = torch.randn(nseq, length, generator=g)
    h0 = torch.randn(nseq, generator=g)
    return a, b, h0


def reference(a, b, h0):
    a64, b64 = a.numpy(), b.numpy()
    h0v = np.zeros(a.shape[0]) if h0 is None else h0.numpy().astype(np.float64)
    big = a.shape[1] > 200_000
    rows = [(native.linear_scan(a64[k], b64[k], float(h0v[k])) if big else
             oracle.linear_scan(a64[k], b64[k], float(h0v[k]))) for k in range(a.shape[0])]
    return np.stack(rows)


def run(a, b, h0):
    dev = need_gpu()
    h, last = ssm.linear_scan_batched(a.to(dev), b.to(dev),
                                      None if h0 is None else h0.to(dev))
    torch.cuda.synchronize()
    return h.cpu().numpy(), last.cpu().numpy()


# sequence lengths below, at and across the lane chunk (4), row (256), wave
# (768), the batched tile (8448) and superblock (64 tiles), and 8192; sequence
# counts from 1 to thousands
SHAPES = [(1, 1), (3, 1), (1000, 1), (5, 2), (7, 3), (9, 4), (4, 5), (33, 255), (17, 256),
          (6, 257), (11, 767), (10, 768), (9, 769), (3, 8191), (2, 8192), (5, 8193),
          (3, 8447), (2, 8448), (4, 8449), (4096, 64), (1024, 1000), (2, 64 * 8448 + 3),
          (1, 64 * 8448), (2, 64 * 8192 + 3), (1, 100003)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}" for s in SHAPES])
def test_batched_shapes(shape):
    nseq, length = shape
    say(f"batched {nseq} x {length}")
    a, b, h0 = inputs(nseq, length, seed=nseq * 7 + length)
    h, last = run(a, b, h0)
    ref = reference(a, b, h0)
    assert_close(h, ref, TOL, f"{nseq}x{length}")
    assert np.array_equal(last, h[:, -1])


def test_batched_without_h0_starts_from_zero():
    a, b, _ = inputs(50, 777, seed=3)
    h, _ = run(a, b, None)
    assert_close(h, reference(a, b, None), TOL, "h0 = None")


def test_batched_one_sequence_matches_single_scan():
    """nseq = 1 is the plain recurrence; compare with ssm_linear_scan (both
    within tolerance of the oracle, and close to each other)."""
    a, b, h0 = inputs(1, 300001, seed=11)
    hb, _ = run(a, b, h0)
    dev = need_gpu()
    hs = ssm.linear_scan(a[0].to(dev), b[0].to(dev), float(h0[0])).cpu().numpy()
    assert_close(hb[0], hs, TOL, "batched vs single")


def test_batched_sequences_are_isolated():
    """inf and NaN inside one sequence stay there: every sequence, those
    holding the values included, matches the oracle run on it alone."""
    say("batched isolation of non-finite values")
    a, b, h0 = inputs(8, 5000, seed=21)
    b[2, 100] = float("inf")
    b[5, 4999] = float("nan")  # last element: h_last[5] is NaN, sequence 6 is not
    h, last = run(a, b, h0)
    ref = reference(a, b, h0)
    assert_same_nonfinite(h, ref, TOL, "all sequences")
    assert np.isnan(last[5]) and np.isfinite(last[6])


def test_batched_integer_exact():
    """a in {0, 1} and small integer b, h0: every value is an exact small
    integer, so any association must give the oracle's result exactly."""
    g = torch.Generator().manual_seed(5)
    nseq, length = 300, 3000
    a = (torch.rand(nseq, length, generator=g) < 0.995).float()
    b = torch.randint(-4, 5, (nseq, length), generator=g).float()
    h0 = torch.randint(-3, 4, (nseq,), generator=g).float()
    h, last = run(a, b, h0)
    assert np.array_equal(h.astype(np.float64), reference(a, b, h0))


def test_batched_deterministic():
    """100 runs bit for bit, at the bench's batched shape (4096 x 32768, 2^27
    elements)."""
    say("batched determinism 100 runs, 4096 x 32768")
    dev = need_gpu()
    a, b, h0 = (t.to(dev) for t in inputs(4096, 32768, seed=8))
    first, _ = ssm.linear_scan_batched(a, b, h0)
    out = torch.empty_like(first)
    mismatches = 0
    for _ in range(99):
        ssm.linear_scan_batched(a, b, h0, out=out)
        if not torch.equal(out.view(torch.int32), first.view(torch.int32)):
            mismatches += 1
    torch.cuda.synchronize()
    say(f"  mismatching runs: {mismatches}")
    assert mismatches == 0
