"""Calls on several HIP streams at once: each (device, stream) has its own
cached workspace (tickets, status words, chunk aggregates), so concurrent
scans on different streams neither share nor race on it, and each result is
bit for bit the one the same call gives alone."""
import pytest
import torch

import mamba_s6_selective_amd as ssm
from gpu_util import need_gpu, say
from mamba_s6_selective_amd.workloads import linear_inputs, s6_inputs

pytestmark = pytest.mark.gpu


def test_linear_scans_on_two_streams_match_serial():
    dev = need_gpu()
    say("linear scans on two streams at once")
    a1, b1 = (t.to(dev) for t in linear_inputs((1 << 22) + 5, seed=11, a_lo=0.5, a_hi=1.0))
    a2, b2 = (t.to(dev) for t in linear_inputs((1 << 23) + 3, seed=12, a_lo=0.5, a_hi=1.0))
    ref1 = ssm.linear_scan(a1, b1, 0.5)
    ref2 = ssm.linear_scan(a2, b2, -0.25)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    outs = []
    for _ in range(6):
        with torch.cuda.stream(s1):
            h1 = ssm.linear_scan(a1, b1, 0.5)
        with torch.cuda.stream(s2):
            h2 = ssm.linear_scan(a2, b2, -0.25)
        outs.append((h1, h2))
    torch.cuda.synchronize()
    for h1, h2 in outs:
        assert torch.equal(h1.view(torch.int32), ref1.view(torch.int32))
        assert torch.equal(h2.view(torch.int32), ref2.view(torch.int32))


def test_s6_scans_on_two_streams_match_serial():
    dev = need_gpu()
    say("S6 scans on two streams at once")
    cases = [(s6_inputs(2, 3000, 256, 16, seed=21, dtype="bf16"), "bidir"),
             (s6_inputs(4, 1500, 320, 16, seed=22, dtype="f32"), "fwd")]
    tens = [[x.to(dev) for x in (i.u, i.delta, i.A, i.B, i.C, i.D)] for i, _ in cases]
    refs = [ssm.selective_scan_fwd(*t, direction=d) for t, (_, d) in zip(tens, cases)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for _ in range(4):
        ys = []
        for s, t, (_, d) in zip(streams, tens, cases):
            with torch.cuda.stream(s):
                ys.append(ssm.selective_scan_fwd(*t, direction=d))
        outs.append(ys)
    torch.cuda.synchronize()
    for ys in outs:
        for y, ref in zip(ys, refs):
            assert torch.equal(y.view(torch.int32), ref.view(torch.int32))


def test_calls_after_release_workspace():
    """ssm_release_workspace frees every cached workspace (after waiting for
    the work that uses it); later calls allocate afresh and give the same
    results bit for bit."""
    dev = need_gpu()
    say("calls after releasing the workspaces")
    a, b = (t.to(dev) for t in linear_inputs(300001, seed=31, a_lo=0.5, a_hi=1.0))
    inp = s6_inputs(2, 2000, 128, 16, seed=32, dtype="bf16")
    t6 = [x.to(dev) for x in (inp.u, inp.delta, inp.A, inp.B, inp.C, inp.D)]
    h_ref = ssm.linear_scan(a, b, 1.0)
    y_ref = ssm.selective_scan_fwd(*t6, direction="bidir")
    torch.cuda.synchronize()
    for _ in range(3):
        ssm.release_workspace()
        h = ssm.linear_scan(a, b, 1.0)
        y = ssm.selective_scan_fwd(*t6, direction="bidir")
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), h_ref.view(torch.int32))
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
