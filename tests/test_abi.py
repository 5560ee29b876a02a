"""CPU-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import re
from pathlib import Path

import pytest

import mamba_s6_selective_amd as ssm

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "ssmscan.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("ssm_linear_scan", "ssm_selective_scan_fwd", "ssm_selective_scan_fwd_bf16"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ssm.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in ssm.SIGNATURES, f"binding has no signature for {name}"


def test_status_strings():
    lib = ssm.load_library()
    assert lib.ssm_status_string(0) == b"ok"
    assert lib.ssm_status_string(-1) == b"invalid argument"
    assert lib.ssm_status_string(12345) == b"unknown status code"


# Argument errors are detected on the host before any HIP call, so they can be
# exercised without a GPU. Pointers below are never dereferenced.
FAKE = 0x1000          # 16-byte aligned, never dereferenced
FAKE_MISALIGNED = 0x1004


def test_linear_scan_argument_errors():
    lib = ssm.load_library()
    assert lib.ssm_linear_scan(None, None, 0.0, None, 0, None) == ssm.SSM_OK
    assert lib.ssm_linear_scan(FAKE, FAKE, 0.0, FAKE, -1, None) == ssm.SSM_ERR_INVALID_ARG
    assert b"n must be" in lib.ssm_last_error()
    assert lib.ssm_linear_scan(None, FAKE, 0.0, FAKE, 5, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_linear_scan(FAKE, FAKE_MISALIGNED, 0.0, FAKE, 5, None) == \
        ssm.SSM_ERR_INVALID_ARG
    assert b"aligned" in lib.ssm_last_error()
    # beyond three levels of 64 tiles of 8192 elements
    assert lib.ssm_linear_scan(FAKE, FAKE, 0.0, FAKE, (1 << 31) + 1, None) == \
        ssm.SSM_ERR_UNSUPPORTED


@pytest.mark.parametrize("fn_name", ["ssm_selective_scan_fwd", "ssm_selective_scan_fwd_bf16"])
def test_s6_argument_errors(fn_name):
    lib = ssm.load_library()
    fn = getattr(lib, fn_name)
    P = [FAKE] * 7
    # zero-sized problems are no-ops
    assert fn(*P, 0, 10, 8, 16, 0, None) == ssm.SSM_OK
    assert fn(*[None] * 7, 2, 0, 8, 16, 0, None) == ssm.SSM_OK
    # negative sizes / bad direction
    assert fn(*P, -1, 10, 8, 16, 0, None) == ssm.SSM_ERR_INVALID_ARG
    assert fn(*P, 1, 10, 8, 16, 3, None) == ssm.SSM_ERR_INVALID_ARG
    assert fn(*P, 1, 10, 8, 16, -1, None) == ssm.SSM_ERR_INVALID_ARG
    # unsupported state sizes
    assert fn(*P, 1, 10, 8, 17, 0, None) == ssm.SSM_ERR_UNSUPPORTED
    assert fn(*P, 1, 10, 8, 0, 0, None) == ssm.SSM_ERR_UNSUPPORTED
    # null / misaligned pointers with work to do
    bad = list(P)
    bad[3] = None
    assert fn(*bad, 1, 10, 8, 16, 0, None) == ssm.SSM_ERR_INVALID_ARG
    bad = list(P)
    bad[6] = FAKE_MISALIGNED
    assert fn(*bad, 1, 10, 8, 16, 0, None) == ssm.SSM_ERR_INVALID_ARG


def test_copy_argument_errors():
    lib = ssm.load_library()
    assert lib.ssm_copy_f32(None, None, 0, None) == ssm.SSM_OK
    assert lib.ssm_copy_f32(FAKE, None, 4, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_copy_f32(FAKE, FAKE, -4, None) == ssm.SSM_ERR_INVALID_ARG


def test_stream_mul_argument_errors():
    lib = ssm.load_library()
    A, B, H = 0x100000, 0x200000, 0x300000
    assert lib.ssm_stream_mul_f32(None, None, None, 0, None) == ssm.SSM_OK
    assert lib.ssm_stream_mul_f32(A, B, None, 4, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_stream_mul_f32(A, B, H, -4, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_stream_mul_f32(A + 4, B, H, 4, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_stream_mul_f32(A, B, B + 16, 16, None) == ssm.SSM_ERR_INVALID_ARG
    assert b"overlaps" in lib.ssm_last_error()
    assert lib.ssm_stream_mul_f32(A, B, H, (1 << 40) + 1, None) == ssm.SSM_ERR_UNSUPPORTED


def test_binding_rejects_host_tensors():
    import torch
    a = torch.ones(8)
    with pytest.raises(ValueError):
        ssm.linear_scan(a, a)


@pytest.mark.parametrize("name", ["ssm_linear_scan_3pass", "ssm_linear_scan_hs"])
def test_linear_scan_3pass_argument_errors(name):
    lib = ssm.load_library()
    f = getattr(lib, name)
    assert f(None, None, 0.0, None, 0, None) == ssm.SSM_OK
    assert f(FAKE, FAKE, 0.0, FAKE, -1, None) == ssm.SSM_ERR_INVALID_ARG
    assert f(FAKE, None, 0.0, FAKE, 5, None) == ssm.SSM_ERR_INVALID_ARG
    assert f(FAKE, FAKE, 0.0, FAKE_MISALIGNED, 5, None) == ssm.SSM_ERR_INVALID_ARG
    assert b"aligned" in lib.ssm_last_error()
    assert f(FAKE, FAKE, 0.0, FAKE, (1 << 31) + 1, None) == ssm.SSM_ERR_UNSUPPORTED


def test_linear_scan_batched_argument_errors():
    lib = ssm.load_library()
    f = lib.ssm_linear_scan_batched
    assert f(None, None, None, None, None, 0, 10, None) == ssm.SSM_OK
    assert f(None, None, None, None, None, 10, 0, None) == ssm.SSM_OK
    assert f(FAKE, FAKE, None, FAKE, None, -1, 10, None) == ssm.SSM_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, FAKE, None, 10, -1, None) == ssm.SSM_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, None, None, 2, 3, None) == ssm.SSM_ERR_INVALID_ARG
    assert f(FAKE_MISALIGNED, FAKE, None, FAKE, None, 2, 3, None) == ssm.SSM_ERR_INVALID_ARG
    assert f(FAKE, FAKE, None, FAKE, None, 1 << 20, (1 << 11) + 1, None) == \
        ssm.SSM_ERR_UNSUPPORTED


def test_selective_scan_ex_argument_errors():
    lib = ssm.load_library()
    f = lib.ssm_selective_scan_fwd_ex
    args = [FAKE] * 8
    assert f(*args, 1, 8, 4, 16, 0, 4, None) == ssm.SSM_ERR_INVALID_ARG   # unknown flag
    assert b"flag" in lib.ssm_last_error()
    assert f(*args, 1, 8, 4, 16, 0, 0, None) == ssm.SSM_ERR_INVALID_ARG   # bias w/o softplus
    assert b"delta_bias" in lib.ssm_last_error()
    no_bias = [FAKE, FAKE, None] + [FAKE] * 5
    assert f(*no_bias, 1, 8, 4, 17, 0, ssm.SSM_FLAG_DELTA_SOFTPLUS, None) == \
        ssm.SSM_ERR_UNSUPPORTED
    assert f(*no_bias, 1, 8, 4, 16, 3, ssm.SSM_FLAG_DELTA_SOFTPLUS, None) == \
        ssm.SSM_ERR_INVALID_ARG
    assert f(*no_bias, 0, 8, 4, 16, 0, ssm.SSM_FLAG_DELTA_SOFTPLUS, None) == ssm.SSM_OK
    mis = [FAKE, FAKE, FAKE_MISALIGNED] + [FAKE] * 5
    assert f(*mis, 1, 8, 4, 16, 0, ssm.SSM_FLAG_DELTA_SOFTPLUS, None) == ssm.SSM_ERR_INVALID_ARG


def test_binding_rejects_overlapping_outputs():
    """Outputs may not share memory with inputs (the kernels read inputs after
    writing outputs); disjoint views of one buffer are fine."""
    import torch
    a, b = torch.zeros(16), torch.zeros(16)
    ssm._same_device(a=a, b=b, out=torch.zeros(16))
    ssm._same_device(a=a[:8], b=b, out=a[8:])
    for out in (a, a[4:12], b[15:]):
        with pytest.raises(ValueError):
            ssm._same_device(a=a, b=b, out=out)
    ssm._same_device(a=a, b=b, out=torch.zeros(4), h_last=torch.zeros(4))
    h = torch.zeros(8)
    with pytest.raises(ValueError):  # two outputs in one buffer
        ssm._same_device(a=a, b=b, out=h, h_last=h[3:5])


def test_outputs_overlapping_inputs_are_rejected():
    """The library checks output ranges against input ranges from the
    pointers and sizes, before any HIP call (nothing is dereferenced)."""
    lib = ssm.load_library()
    A, B = 0x100000, 0x200000   # 1 MiB apart
    # linear: h = a, h inside b, h just past the end of a (fine)
    assert lib.ssm_linear_scan(A, B, 0.0, A, 16, None) == ssm.SSM_ERR_INVALID_ARG
    assert b"overlaps" in lib.ssm_last_error()
    assert lib.ssm_linear_scan(A, B, 0.0, B + 16, 16, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_linear_scan_3pass(A, B, 0.0, A + 48, 16, None) == ssm.SSM_ERR_INVALID_ARG
    assert lib.ssm_copy_f32(A, A + 32, 16, None) == ssm.SSM_ERR_INVALID_ARG
    # batched: h_last inside h
    assert lib.ssm_linear_scan_batched(A, B, None, 0x300000, 0x300000 + 64, 4, 8, None) == \
        ssm.SSM_ERR_INVALID_ARG
    # S6: y on top of B (bf16 B is smaller than the fp32 y)
    P = [0x1000000 * (k + 1) for k in range(7)]
    bad = list(P)
    bad[6] = P[3] + 32
    for fn in (lib.ssm_selective_scan_fwd, lib.ssm_selective_scan_fwd_bf16):
        assert fn(*bad, 1, 10, 8, 16, 0, None) == ssm.SSM_ERR_INVALID_ARG
        assert b"overlaps" in lib.ssm_last_error()
