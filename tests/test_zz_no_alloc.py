"""The allocation-free linear scan (ssm_linear_scan_noalloc) against the
ordinary entry point (ssm_linear_scan), through the C ABI: the same kernel
and tile shapes, so the outputs must be equal bit for bit. Two calls in a
row, the second smaller (the shared status memory keeps the first call's
contents), then a larger one again, and a size beyond the status memory is
refused."""
import ctypes

import numpy as np
import pytest
import torch

import mamba_s6_selective_amd as ssm
from gpu_util import need_gpu, say
from mamba_s6_selective_amd.workloads import linear_inputs

pytestmark = pytest.mark.gpu


def _noalloc(lib, a, b, h0, out):
    return lib.ssm_linear_scan_noalloc(a.data_ptr(), b.data_ptr(), ctypes.c_float(h0),
                                       out.data_ptr(), a.numel(),
                                       torch.cuda.current_stream().cuda_stream)


def _plain(lib, a, b, h0, out):
    return lib.ssm_linear_scan(a.data_ptr(), b.data_ptr(), ctypes.c_float(h0), out.data_ptr(),
                               a.numel(), torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("sizes", [(3_000_017, 70_001, 8192 * 300 + 5), (1 << 27, 12345, 1)])
def test_noalloc_equals_linear_scan(sizes):
    dev = need_gpu()
    lib = ssm.load_library()
    for k, n in enumerate(sizes):
        say(f"noalloc call {k}: n={n}")
        a, b = (t.to(dev) for t in linear_inputs(n, seed=700 + k, a_lo=0.5, a_hi=1.0))
        h_ref = torch.full_like(a, float("nan"))
        h_na = torch.full_like(a, float("nan"))
        assert _plain(lib, a, b, 0.5, h_ref) == 0
        assert _noalloc(lib, a, b, 0.5, h_na) == 0, lib.ssm_last_error()
        torch.cuda.synchronize()
        same = torch.equal(h_na.view(torch.int32), h_ref.view(torch.int32))
        say(f"  bitwise equal: {same}")
        assert same


def test_noalloc_refuses_beyond_its_memory():
    lib = ssm.load_library()
    big = (1 << 31) + 1
    rc = lib.ssm_linear_scan_noalloc(0x1000, 0x2000000000, ctypes.c_float(0.0), 0x4000000000,
                                     big, None)
    assert rc == ssm.SSM_ERR_UNSUPPORTED
    assert b"2^31" in lib.ssm_last_error()


def test_noalloc_in_a_recorded_graph():
    """Nothing to allocate, so even a first call can be recorded; every replay
    equals the eager result bit for bit."""
    dev = need_gpu()
    a, b = (t.to(dev) for t in linear_inputs(500_003, seed=77, a_lo=0.5, a_hi=1.0))
    ref = ssm.linear_scan(a, b, -0.25)
    y = torch.empty_like(a)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        ssm.linear_scan_noalloc(a, b, -0.25, out=y)
    for r in range(4):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), r
