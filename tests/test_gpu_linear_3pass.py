"""GPU parity of the three-pass linear scan (work-efficient and Hillis-Steele
local passes) against the float64 oracle.

Same bar as the single-pass scan: max |err| <= 1e-4 * (1 + |ref|) for fp32,
bitwise identical from run to run.
"""
import numpy as np
import pytest
import torch

import mamba_s6_selective_amd as ssm
import oracle
from gpu_util import assert_close, need_gpu, say
from mamba_s6_selective_amd.workloads import linear_inputs, linear_workload_inputs
from oracle import native
from test_gpu_linear import EDGE_N

pytestmark = pytest.mark.gpu
TOL = 1e-4


KINDS = {"3pass": lambda *a, **k: ssm.linear_scan_3pass(*a, **k),
         "hs": lambda *a, **k: ssm.linear_scan_hs(*a, **k)}


def run3(a, b, h0=0.0, kind="3pass"):
    dev = need_gpu()
    h = KINDS[kind](a.to(dev), b.to(dev), h0)
    torch.cuda.synchronize()
    return h.cpu()


@pytest.mark.parametrize("kind", sorted(KINDS))
@pytest.mark.parametrize("n", EDGE_N)
def test_3pass_edge_sizes(n, kind):
    say(f"{kind} edge n={n}")
    a, b = linear_inputs(n, seed=900 + n, a_lo=0.5, a_hi=1.0)
    h0 = -1.25
    if n > 1_000_000:
        ref = native.linear_scan(a.numpy(), b.numpy(), h0)
    else:
        ref = oracle.linear_scan(a.numpy(), b.numpy(), h0)
    assert_close(run3(a, b, h0, kind).numpy(), ref, TOL, f"{kind} n={n}")


def test_3pass_zero_length_is_noop():
    dev = need_gpu()
    a = torch.empty(0, device=dev)
    assert ssm.linear_scan_3pass(a, a, 1.0).numel() == 0


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_3pass_prefix_sum_exact(kind):
    say(f"{kind} a=1 integer prefix sum, exact")
    n = 3 * 1024 * 1024 + 5
    g = torch.Generator().manual_seed(15)
    b = torch.randint(-8, 9, (n,), generator=g).float()
    a = torch.ones(n)
    ref = -2.0 + np.cumsum(b.numpy().astype(np.float64))
    assert np.array_equal(run3(a, b, -2.0, kind).numpy().astype(np.float64), ref)


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_3pass_signed_coefficients(kind):
    a, b = linear_inputs(300001, seed=78, a_lo=-1.0, a_hi=1.0)
    ref = oracle.linear_scan(a.numpy(), b.numpy(), 2.0)
    assert_close(run3(a, b, 2.0, kind).numpy(), ref, TOL, f"{kind} signed")


def test_hs_full_size_workload_and_determinism():
    say("linear-n134217728 Hillis-Steele three-pass vs C oracle, 5 repeated runs")
    dev = need_gpu()
    a, b = linear_workload_inputs("linear-n134217728")
    ad, bd = a.to(dev), b.to(dev)
    first = ssm.linear_scan_hs(ad, bd, 0.0)
    out = torch.empty_like(first)
    for _ in range(4):
        ssm.linear_scan_hs(ad, bd, 0.0, out=out)
        assert torch.equal(out.view(torch.int32), first.view(torch.int32))
    torch.cuda.synchronize()
    ref = native.linear_scan(a.numpy(), b.numpy(), 0.0)
    assert_close(first.cpu().numpy(), ref, TOL, "linear-n134217728 hs")


def test_3pass_full_size_workload_and_determinism():
    say("linear-n134217728 three-pass vs C oracle, 10 repeated runs")
    dev = need_gpu()
    a, b = linear_workload_inputs("linear-n134217728")
    ad, bd = a.to(dev), b.to(dev)
    first = ssm.linear_scan_3pass(ad, bd, 0.0)
    out = torch.empty_like(first)
    for _ in range(9):
        ssm.linear_scan_3pass(ad, bd, 0.0, out=out)
        assert torch.equal(out.view(torch.int32), first.view(torch.int32))
    torch.cuda.synchronize()
    ref = native.linear_scan(a.numpy(), b.numpy(), 0.0)
    assert_close(first.cpu().numpy(), ref, TOL, "linear-n134217728 3-pass")


@pytest.mark.parametrize("kind", sorted(KINDS))
def test_3pass_above_2_27_uncached_carry_exact(kind):
    """n = 2^28 + 5*8192 + 3: more than 16384 tiles, so the carry pass's
    waves hold more than one batch of 16 rows and re-scan them on the second
    walk, and the last tile is ragged. a = 1 and b = 1 at 1000 seeded
    positions (0 elsewhere): h[i] = h0 + (ones at positions <= i) exactly in
    fp32 whatever the grouping. Checked at every tile end, at the ones and
    just before them, at the last element and at 2^20 seeded positions."""
    n = (1 << 28) + 5 * 8192 + 3
    say(f"{kind} n={n}: a = 1, sparse integer b")
    dev = need_gpu()
    g = torch.Generator().manual_seed(2028)
    pos = np.unique(torch.randint(0, n, (1000,), generator=g).numpy().astype(np.int64))
    a = torch.ones(n, device=dev)
    b = torch.zeros(n, device=dev)
    b[torch.from_numpy(pos).to(dev)] = 1.0
    h = KINDS[kind](a, b, 0.5)
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
