"""Calls recorded in a HIP graph and replayed: once a first call on the
capture stream has sized that stream's workspace, a call enqueues kernels
only (no allocation, no memset), and every replay, with eager work between
replays, equals the eager result bit for bit. The single-pass linear scans
take their status-word epoch from the device, so replays and eager calls on
the same workspace keep getting fresh epochs; a short epoch cycle drives the
clearing of the status words that ends each cycle through many wraps."""
import os

import pytest
import torch

import mamba_s6_selective_amd as ssm
from gpu_util import need_gpu, say
from mamba_s6_selective_amd.workloads import linear_inputs, s6_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("direction,fused", [("fwd", False), ("bidir", False), ("fwd", True)])
def test_s6_graph_replay(direction, fused):
    dev = need_gpu()
    say(f"S6 graph replay ({direction}{', fused softplus' if fused else ''})")
    inp = s6_inputs(2, 3000, 256, 16, seed=41, dtype="bf16")
    t = [x.to(dev) for x in (inp.u, inp.delta_pre if fused else inp.delta, inp.A, inp.B,
                             inp.C, inp.D)]
    kw = {"direction": direction, "delta_softplus": fused}
    ref = ssm.selective_scan_fwd(*t, **kw)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(ref)
    with torch.cuda.stream(s):
        ssm.selective_scan_fwd(*t, out=y, **kw)  # sizes the workspace of s
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ssm.selective_scan_fwd(*t, out=y, **kw)
    torch.cuda.synchronize()
    for k in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # eager work between replays
        e = ssm.selective_scan_fwd(*t, **kw)
        torch.cuda.synchronize()
        assert torch.equal(e.view(torch.int32), ref.view(torch.int32))
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), k


TILE = 8192  # elements per tile of the single-pass scan (the batched form: 8448)


def _bits(x):
    return x.view(torch.int32)


@pytest.mark.parametrize("batched", [False, True])
def test_linear_graph_replay(batched):
    dev = need_gpu()
    say(f"linear scan graph replay ({'batched' if batched else 'single'})")
    n = 130 * TILE + 777 if not batched else 37 * (3 * 8448 + 5)
    ins = [tuple(t.to(dev) for t in linear_inputs(n, seed=s, a_lo=0.5, a_hi=1.0))
           for s in (51, 52)]
    a, b = (x.clone() for x in ins[0])
    nseq = 37
    h0 = torch.linspace(-1, 1, nseq, device=dev)
    last = torch.empty(nseq, device=dev)

    def run(a_, b_, out=None):
        if batched:  # h, with each sequence's last value appended
            h, hl = ssm.linear_scan_batched(a_.view(nseq, -1), b_.view(nseq, -1), h0,
                                            out=None if out is None else out[:n].view(nseq, -1),
                                            h_last=last)
            if out is None:
                out = torch.empty(n + nseq, device=dev)
                out[:n] = h.view(-1)
            out[n:] = hl
            return out
        return ssm.linear_scan(a_, b_, 0.25, out=out)

    refs = [run(*x).clone() for x in ins]
    small_a, small_b = (t.to(dev) for t in linear_inputs(3 * TILE + 17, seed=53))
    small_ref = ssm.linear_scan(small_a, small_b, -0.5)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(refs[0])  # batched: h, then the last values
    with torch.cuda.stream(s):
        run(a, b, out=y)  # sizes the workspace of s
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(a, b, out=y)
    torch.cuda.synchronize()
    for k in range(6):
        src = ins[k % 2]
        a.copy_(src[0])
        b.copy_(src[1])
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
            if k % 3 == 2:
                g.replay()  # back to back on one stream
        s.synchronize()
        assert torch.equal(_bits(y), _bits(refs[k % 2])), k
        with torch.cuda.stream(s):  # an eager call on the same workspace between replays
            e = ssm.linear_scan(small_a, small_b, -0.5)
        s.synchronize()
        assert torch.equal(_bits(e), _bits(small_ref)), k


def test_linear_epoch_cycle_clears_status_words():
    """With a cycle of c epochs every c-th launch on a workspace clears its
    status words. A large launch followed by small ones leaves words of its
    epoch on tiles the small ones never touch; the next large launch with that
    epoch would read them as current had they not been cleared."""
    dev = need_gpu()
    big = 300 * TILE + 1234
    a_big, b_big = (t.to(dev) for t in linear_inputs(big, seed=61, a_lo=0.5, a_hi=1.0))
    a_big2, b_big2 = (t.to(dev) for t in linear_inputs(big, seed=62, a_lo=0.5, a_hi=1.0))
    a_sm, b_sm = (t.to(dev) for t in linear_inputs(5 * TILE + 3, seed=63))
    nseq = 24
    a_bt, b_bt = (t.to(dev) for t in linear_inputs(nseq * 40000, seed=64))
    h0 = torch.linspace(-2, 2, nseq, device=dev)
    calls = {
        "big": lambda: ssm.linear_scan(a_big, b_big, 1.5),
        "big2": lambda: ssm.linear_scan(a_big2, b_big2, -1.0),
        "small": lambda: ssm.linear_scan(a_sm, b_sm, 0.0),
        "batched": lambda: torch.cat([x.view(-1) for x in ssm.linear_scan_batched(
            a_bt.view(nseq, -1), b_bt.view(nseq, -1), h0)]),
    }
    seq = ["big", "small", "small", "big", "big2", "small", "batched", "small", "big",
           "small", "small", "small", "big2", "batched", "big", "small", "big"]
    try:
        ssm.release_workspace()
        refs = {k: f().clone() for k, f in calls.items()}
        torch.cuda.synchronize()
        for cycle in (3, 2, 1):
            say(f"linear epoch cycle {cycle}")
            ssm.release_workspace()
            os.environ["SSMSCAN_LINEAR_EPOCH_CYCLE"] = str(cycle)  # read by new workspaces
            outs = [(k, calls[k]()) for k in seq]
            torch.cuda.synchronize()
            for i, (k, h) in enumerate(outs):
                assert torch.equal(_bits(h), _bits(refs[k])), (cycle, i, k)
            if cycle == 2:
                # Replays that end cycles themselves: a recorded large call
                # and eager small calls alternate on one workspace.
                st = torch.cuda.Stream()
                y = torch.empty_like(refs["big"])
                with torch.cuda.stream(st):
                    ssm.linear_scan(a_big, b_big, 1.5, out=y)
                st.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=st):
                    ssm.linear_scan(a_big, b_big, 1.5, out=y)
                torch.cuda.synchronize()
                for r in range(5):
                    y.fill_(float("nan"))
                    torch.cuda.synchronize()
                    with torch.cuda.stream(st):
                        g.replay()
                        hs = ssm.linear_scan(a_sm, b_sm, 0.0) if r % 2 else None
                    st.synchronize()
                    assert torch.equal(_bits(y), _bits(refs["big"])), ("replay", r)
                    if hs is not None:
                        assert torch.equal(_bits(hs), _bits(refs["small"])), ("replay", r)
                del g
    finally:
        ssm.release_workspace()
        os.environ.pop("SSMSCAN_LINEAR_EPOCH_CYCLE", None)


def test_workspace_growth_during_capture_is_refused():
    dev = need_gpu()
    say("workspace growth refused during capture")
    a, b = (t.to(dev) for t in linear_inputs(4 * TILE, seed=71))
    y = torch.empty_like(a)
    inp = s6_inputs(1, 512, 128, 16, seed=72, dtype="f32")
    t = [x.to(dev) for x in (inp.u, inp.delta, inp.A, inp.B, inp.C, inp.D)]
    ys6 = torch.empty(1, 512, 128, device=dev)
    torch.cuda.synchronize()
    for call in (lambda: ssm.linear_scan(a, b, 0.0, out=y),
                 lambda: ssm.selective_scan_fwd(*t, out=ys6)):
        s = torch.cuda.Stream()  # a new stream: no workspace yet
        g = torch.cuda.CUDAGraph()
        with pytest.raises(ssm.SsmScanError) as err:
            with torch.cuda.graph(g, stream=s):
                call()
        assert err.value.code == -1 and "outside graph capture" in str(err.value)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):  # the same call outside capture then works
            call()
        torch.cuda.synchronize()
    ref = ssm.linear_scan(a, b, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(ref))


def test_graph_replay_after_workspace_growth():
    """A larger call on the capture stream moves the stream to a larger
    workspace; the recorded calls keep the workspaces they were recorded
    with, which stay allocated until release_workspace."""
    dev = need_gpu()
    say("graph replay after workspace growth")
    a, b = (t.to(dev) for t in linear_inputs(3 * TILE + 17, seed=81, a_lo=0.5, a_hi=1.0))
    big = 4100 * TILE + 5  # past the smallest linear workspace (4096 tiles)
    a2, b2 = (t.to(dev) for t in linear_inputs(big, seed=82, a_lo=0.5, a_hi=1.0))
    small = s6_inputs(1, 512, 128, 16, seed=83, dtype="f32")
    large = s6_inputs(2, 4096, 512, 16, seed=84, dtype="f32")  # a larger S6 workspace
    ts = [x.to(dev) for x in (small.u, small.delta, small.A, small.B, small.C, small.D)]
    tl = [x.to(dev) for x in (large.u, large.delta, large.A, large.B, large.C, large.D)]
    ref_lin, ref_lin2 = ssm.linear_scan(a, b, 0.5), ssm.linear_scan(a2, b2, -0.5)
    ref_s6, ref_s6l = ssm.selective_scan_fwd(*ts), ssm.selective_scan_fwd(*tl)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    y = torch.empty_like(ref_lin)
    ys6 = torch.empty_like(ref_s6)
    with torch.cuda.stream(s):  # size the stream's workspaces for the small calls
        ssm.linear_scan(a, b, 0.5, out=y)
        ssm.selective_scan_fwd(*ts, out=ys6)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ssm.linear_scan(a, b, 0.5, out=y)
        ssm.selective_scan_fwd(*ts, out=ys6)
    torch.cuda.synchronize()
    for k in range(3):
        with torch.cuda.stream(s):  # larger calls: new workspaces for s (grown on the first)
            h2 = ssm.linear_scan(a2, b2, -0.5)
            yl = ssm.selective_scan_fwd(*tl)
        s.synchronize()
        assert torch.equal(_bits(h2), _bits(ref_lin2)), k
        assert torch.equal(_bits(yl), _bits(ref_s6l)), k
        y.fill_(float("nan"))
        ys6.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert torch.equal(_bits(y), _bits(ref_lin)), k
        assert torch.equal(_bits(ys6), _bits(ref_s6)), k
