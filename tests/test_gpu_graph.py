"""S6 calls recorded in a HIP graph and replayed: once a first call on the
capture stream has sized that stream's workspace, a call enqueues kernels
only (no allocation, no memset), and every replay, with eager work between
replays, equals the eager result bit for bit."""
import pytest
import torch

import mamba_s6_selective_amd as ssm
from gpu_util import need_gpu, say
from mamba_s6_selective_amd.workloads import s6_inputs

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
