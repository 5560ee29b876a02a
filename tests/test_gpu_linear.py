"""GPU parity of the look-back linear scan against the float64 oracle.

Bar: max |err| <= 1e-4 * (1 + |ref|) elementwise for fp32; bitwise identity
across 100 repeated runs (the look-back always folds in the same order).
"""
import hashlib

import numpy as np
import pytest
import torch

import mamba_s6_selective_amd as ssm
import oracle
from gpu_util import assert_close, need_gpu, say
from mamba_s6_selective_amd.workloads import linear_inputs, linear_workload_inputs
from oracle import native

pytestmark = pytest.mark.gpu
TOL = 1e-4


def run(a, b, h0=0.0):
    dev = need_gpu()
    h = ssm.linear_scan(a.to(dev), b.to(dev), h0)
    torch.cuda.synchronize()
    return h.cpu()


def test_linear_n65536_workload():
    say("linear-n65536 (a~U(0.9,1), b~N(0,1), h0=0)")
    a, b = linear_workload_inputs("linear-n65536")
    ref = oracle.linear_scan(a.numpy(), b.numpy(), 0.0)
    assert_close(run(a, b).numpy(), ref, TOL, "linear-n65536")


# sizes straddling lane chunks (4), rows (256), waves (1024; 2048 in the
# three-pass kernel), tiles (8192),
# superblocks (64 tiles) and blocks (4096 tiles)
EDGE_N = [1, 2, 3, 4, 5, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049,
          4095, 4096, 8191, 8192, 8193, 12289, 65537, 100003, 262144 + 77,
          64 * 8192 - 1, 64 * 8192, 64 * 8192 + 1, 65 * 8192 + 3,
          4096 * 8192 - 1, 4096 * 8192 + 5]


@pytest.mark.parametrize("n", EDGE_N)
def test_linear_edge_sizes(n):
    say(f"linear edge n={n}")
    a, b = linear_inputs(n, seed=500 + n, a_lo=0.5, a_hi=1.0)
    h0 = 0.75
    if n > 1_000_000:
        ref = native.linear_scan(a.numpy(), b.numpy(), h0)
    else:
        ref = oracle.linear_scan(a.numpy(), b.numpy(), h0)
    assert_close(run(a, b, h0).numpy(), ref, TOL, f"n={n}")


def test_linear_zero_length_is_noop():
    dev = need_gpu()
    a = torch.empty(0, device=dev)
    assert ssm.linear_scan(a, a, 1.0).numel() == 0


def test_linear_signed_coefficients():
    say("linear signed a ~ U(-1, 1), many tiles")
    a, b = linear_inputs(300000, seed=77, a_lo=-1.0, a_hi=1.0)
    ref = oracle.linear_scan(a.numpy(), b.numpy(), -2.0)
    assert_close(run(a, b, -2.0).numpy(), ref, TOL, "signed")


def test_linear_prefix_sum_exact():
    """a == 1 with small integer b: every partial sum is an integer below 2^24,
    so any association is exact and the result must equal the prefix sum."""
    say("linear a=1 integer prefix sum, exact")
    n = 2 * 1024 * 1024 - 3
    g = torch.Generator().manual_seed(5)
    b = torch.randint(-8, 9, (n,), generator=g).float()
    a = torch.ones(n)
    h = run(a, b, 3.0)
    ref = 3.0 + np.cumsum(b.numpy().astype(np.float64))
    assert np.array_equal(h.numpy().astype(np.float64), ref)


def test_linear_reset_segments_exact():
    """a in {0, 1}, integer b: segmented prefix sums, exact."""
    say("linear a in {0,1} segmented, exact")
    n = 200000
    g = torch.Generator().manual_seed(6)
    a = (torch.rand(n, generator=g) < 0.999).float()
    b = torch.randint(-8, 9, (n,), generator=g).float()
    ref = native.linear_scan(a.numpy(), b.numpy(), 1.0)
    assert np.array_equal(run(a, b, 1.0).numpy().astype(np.float64), ref)


def test_linear_nan_propagates_without_hang():
    say("linear NaN propagation")
    n = 50000
    a, b = linear_inputs(n, seed=9, a_lo=0.5, a_hi=1.0)
    b[20000] = float("nan")
    ref = oracle.linear_scan(a.numpy(), b.numpy(), 0.0)
    assert_close(run(a, b).numpy(), ref, TOL, "nan")


def test_linear_full_size_workload():
    say("linear-n134217728 full size vs C oracle")
    dev = need_gpu()
    a, b = linear_workload_inputs("linear-n134217728")
    h = ssm.linear_scan(a.to(dev), b.to(dev), 0.0)
    torch.cuda.synchronize()
    ref = native.linear_scan(a.numpy(), b.numpy(), 0.0)
    assert_close(h.cpu().numpy(), ref, TOL, "linear-n134217728")


def test_linear_homogeneous_bit_exact_full_size():
    """h is linear in (b, h0), and doubling both doubles every product and
    sum without a new rounding (no value here is near under- or overflow):
    h(a, 2b, 2h0) equals 2 h(a, b, h0) bit for bit at 2^27 elements, however
    the look-back groups the fold."""
    say("linear-n134217728: h(a, 2b, 2h0) == 2 h(a, b, h0)")
    dev = need_gpu()
    a, b = linear_workload_inputs("linear-n134217728")
    a, b = a.to(dev), b.to(dev)
    h1 = ssm.linear_scan(a, b, 0.75)
    h2 = ssm.linear_scan(a, b * 2, 1.5)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(h1).all())
    bad = int((h2 != 2 * h1).sum())
    say(f"  elements not exactly doubled: {bad}")
    assert bad == 0


@pytest.mark.parametrize("n", [1 << 31, (1 << 31) - 4093])
def test_linear_maximum_size_carry_exact(n):
    """n = 2^31, the largest length the single-pass scan accepts (every
    look-back level full: 64 blocks of 64 superblocks of 64 tiles), and the
    same with a ragged last tile, with a = 1 and b = 1 at 1000 seeded
    positions, 0 elsewhere: every carry crosses the whole sequence, and
    h[i] = h0 + (number of ones at positions <= i) exactly in fp32 whatever
    the grouping. Checked at every tile's last element, at the ones and just
    before them, at the last element and at 2^20 seeded positions."""
    say(f"linear maximum size n={n}: a = 1, sparse integer b")
    dev = need_gpu()
    g = torch.Generator().manual_seed(2031)
    pos = np.unique(torch.randint(0, n, (1000,), generator=g).numpy().astype(np.int64))
    a = torch.ones(n, device=dev)
    b = torch.zeros(n, device=dev)
    b[torch.from_numpy(pos).to(dev)] = 1.0
    h = ssm.linear_scan(a, b, 0.5)
    del a, b
    tile = 8192
    idx = np.concatenate([
        np.arange(tile - 1, n, tile, dtype=np.int64), [0, n - 1], pos, np.maximum(pos - 1, 0),
        torch.randint(0, n, (1 << 20,), generator=g).numpy().astype(np.int64)])
    got = h[torch.from_numpy(idx).to(dev)].cpu().numpy()
    del h
    torch.cuda.synchronize()
    expected = 0.5 + np.searchsorted(pos, idx, side="right").astype(np.float64)
    bad = int(np.count_nonzero(got != expected))
    say(f"  {idx.size} positions checked, {bad} differ")
    assert bad == 0


@pytest.mark.parametrize("n", [1 << 27, (1 << 20) + 3])
def test_linear_bitwise_determinism_100_runs(n):
    say(f"linear determinism 100 runs n={n}")
    dev = need_gpu()
    a, b = linear_inputs(n, seed=31, a_lo=0.5, a_hi=1.0)
    a, b = a.to(dev), b.to(dev)
    first = ssm.linear_scan(a, b, 0.5)
    out = torch.empty_like(first)
    mismatches = 0
    for _ in range(99):
        ssm.linear_scan(a, b, 0.5, out=out)
        if not torch.equal(out.view(torch.int32), first.view(torch.int32)):
            mismatches += 1
    torch.cuda.synchronize()
    digest = hashlib.sha256(first.cpu().numpy().tobytes()).hexdigest()[:16]
    say(f"  sha256 {digest}, mismatching runs: {mismatches}")
    assert mismatches == 0


def test_copy_sentinel():
    dev = need_gpu()
    x = torch.randn(1000003, device=dev)
    y = torch.empty_like(x)
    ssm.copy_f32(x, y)
    assert torch.equal(x, y)


@pytest.mark.parametrize("n", [1, 3, 4, 1023, 1024, 1025, 4 * 256 + 3, 1000003, 1 << 22])
def test_stream_mul_exact(n):
    """The bandwidth reference kernel: h = a * b, each product the IEEE fp32
    one (equal to the CPU's), at sizes with 0-3 tail elements and several
    workgroups."""
    say(f"stream mul n={n}")
    dev = need_gpu()
    g = torch.Generator().manual_seed(n)
    a, b = torch.randn(n, generator=g), torch.randn(n, generator=g)
    h = ssm.stream_mul_f32(a.to(dev), b.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(h.cpu(), a * b)
