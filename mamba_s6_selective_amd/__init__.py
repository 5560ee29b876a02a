"""Python binding of libssmscan (HIP, gfx950): argument marshalling only.

Every step of the computation runs in the library's HIP kernels; torch is used
for device memory and for the current stream. There is no CPU fallback: if
libssmscan.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libssmscan.so"

DIRECTIONS = {"fwd": 0, "rev": 1, "bidir": 2}

SSM_FLAG_BF16 = 1
SSM_FLAG_DELTA_SOFTPLUS = 2

SSM_OK = 0
SSM_ERR_INVALID_ARG = -1
SSM_ERR_UNSUPPORTED = -2
SSM_ERR_HIP = -3
SSM_ERR_ALLOC = -4

# Every symbol include/ssmscan.h declares, with its ctypes signature.
_P = ctypes.c_void_p
SIGNATURES = {
    "ssm_linear_scan": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, ctypes.c_int64, _P]),
    "ssm_linear_scan_noalloc": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, ctypes.c_int64, _P]),
    "ssm_linear_scan_3pass": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, ctypes.c_int64, _P]),
    "ssm_linear_scan_hs": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, ctypes.c_int64, _P]),
    "ssm_linear_scan_batched": (ctypes.c_int, [_P] * 5 + [ctypes.c_int64, ctypes.c_int64, _P]),
    "ssm_selective_scan_fwd": (ctypes.c_int, [_P] * 7 + [ctypes.c_int] * 5 + [_P]),
    "ssm_selective_scan_fwd_bf16": (ctypes.c_int, [_P] * 7 + [ctypes.c_int] * 5 + [_P]),
    "ssm_selective_scan_fwd_ex": (ctypes.c_int, [_P] * 8 + [ctypes.c_int] * 5 +
                                  [ctypes.c_uint, _P]),
    "ssm_copy_f32": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "ssm_stream_mul_f32": (ctypes.c_int, [_P, _P, _P, ctypes.c_int64, _P]),
    "ssm_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssm_last_error": (ctypes.c_char_p, []),
    "ssm_release_workspace": (ctypes.c_int, []),
}

_lib = None


class SsmScanError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libssmscan error {code}: {msg}")
        self.code = code


def load_library():
    """Load libssmscan.so (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m mamba_s6_selective_amd.build`")
    lib = ctypes.CDLL(str(LIB_PATH))
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code: int):
    if code != SSM_OK:
        lib = load_library()
        raise SsmScanError(code, lib.ssm_last_error().decode() or
                           lib.ssm_status_string(code).decode())


def _stream(tensor) -> int:
    import torch
    return torch.cuda.current_stream(tensor.device).cuda_stream


def _dev_tensor(t, name, dtypes):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(**tensors):
    """All given tensors (None skipped) on one device, and each output
    (names starting with "out" or "h_last") sharing no memory with any input."""
    items = [(k, t) for k, t in tensors.items() if t is not None]
    dev = items[0][1].device
    for k, t in items:
        if t.device != dev:
            raise ValueError(f"{k} is on {t.device}, expected {dev}")

    def span(t):
        start = t.data_ptr()
        return start, start + t.numel() * t.element_size()

    outs = [(k, t) for k, t in items if k.startswith("out") or k == "h_last"]
    ins = [(k, t) for k, t in items if not (k.startswith("out") or k == "h_last")]
    for ko, o in outs:
        o0, o1 = span(o)
        for ki, i in ins + [x for x in outs if x[0] != ko]:
            i0, i1 = span(i)
            if o0 < i1 and i0 < o1:
                raise ValueError(f"{ko} overlaps {ki}")


def _linear_args(a, b, out):
    import torch
    _dev_tensor(a, "a", (torch.float32,))
    _dev_tensor(b, "b", (torch.float32,))
    if a.shape != b.shape or a.dim() != 1:
        raise ValueError("a and b must be 1-D and of equal length")
    if out is None:
        out = torch.empty_like(a)
    else:
        _dev_tensor(out, "out", (torch.float32,))
        if out.shape != a.shape:
            raise ValueError("out must match a")
    _same_device(a=a, b=b, out=out)
    return out


def linear_scan_batched(a, b, h0=None, out=None, h_last=None):
    """Independent recurrences over the rows of 2-D (nseq, len) fp32 device
    tensors: h[k][t] = a[k][t]*h[k][t-1] + b[k][t], h[k][-1] = h0[k] (0 when
    h0 is None). Returns (h, h_last) with h_last[k] = h[k][len-1]."""
    import torch
    lib = load_library()
    _dev_tensor(a, "a", (torch.float32,))
    _dev_tensor(b, "b", (torch.float32,))
    if a.shape != b.shape or a.dim() != 2:
        raise ValueError("a and b must be 2-D (nseq, len) and of equal shape")
    nseq, length = a.shape
    if h0 is not None:
        _dev_tensor(h0, "h0", (torch.float32,))
        if h0.shape != (nseq,):
            raise ValueError("h0 must have shape (nseq,)")
    if out is None:
        out = torch.empty_like(a)
    else:
        _dev_tensor(out, "out", (torch.float32,))
        if out.shape != a.shape:
            raise ValueError("out must match a")
    if h_last is None:
        h_last = torch.empty(nseq, dtype=torch.float32, device=a.device)
    else:
        _dev_tensor(h_last, "h_last", (torch.float32,))
        if h_last.shape != (nseq,):
            raise ValueError("h_last must have shape (nseq,)")
    _same_device(a=a, b=b, h0=h0, out=out, h_last=h_last)
    with torch.cuda.device(a.device):
        _check(lib.ssm_linear_scan_batched(
            a.data_ptr(), b.data_ptr(), None if h0 is None else h0.data_ptr(), out.data_ptr(),
            h_last.data_ptr(), nseq, length, _stream(a)))
    return out, h_last


def linear_scan_3pass(a, b, h0: float = 0.0, out=None):
    """The same recurrence by the three-pass design (28 B/element of traffic)."""
    import torch
    lib = load_library()
    out = _linear_args(a, b, out)
    with torch.cuda.device(a.device):
        _check(lib.ssm_linear_scan_3pass(a.data_ptr(), b.data_ptr(), float(h0),
                                         out.data_ptr(), a.numel(), _stream(a)))
    return out


def linear_scan_hs(a, b, h0: float = 0.0, out=None):
    """The same recurrence, three passes with a register-resident
    Hillis-Steele local pass."""
    import torch
    lib = load_library()
    out = _linear_args(a, b, out)
    with torch.cuda.device(a.device):
        _check(lib.ssm_linear_scan_hs(a.data_ptr(), b.data_ptr(), float(h0),
                                      out.data_ptr(), a.numel(), _stream(a)))
    return out


def linear_scan(a, b, h0: float = 0.0, out=None):
    """h[t] = a[t]*h[t-1] + b[t], h[-1] = h0 (fp32, 1-D device tensors)."""
    import torch
    lib = load_library()
    out = _linear_args(a, b, out)
    with torch.cuda.device(a.device):
        _check(lib.ssm_linear_scan(a.data_ptr(), b.data_ptr(), float(h0), out.data_ptr(),
                                   a.numel(), _stream(a)))
    return out


def linear_scan_noalloc(a, b, h0: float = 0.0, out=None):
    """linear_scan through the library's allocation-free entry point (status
    memory inside the library; calls on one GPU must not overlap)."""
    import torch
    lib = load_library()
    out = _linear_args(a, b, out)
    with torch.cuda.device(a.device):
        _check(lib.ssm_linear_scan_noalloc(a.data_ptr(), b.data_ptr(), float(h0),
                                           out.data_ptr(), a.numel(), _stream(a)))
    return out


def selective_scan_fwd(u, delta, A, B, C, D, direction: str = "fwd", out=None,
                       delta_bias=None, delta_softplus: bool = False):
    """S6 scan. u, delta: (batch, L, d); A: (d, N) fp32; B, C: (batch, L, N);
    D: (d,) fp32. u, delta, B, C all fp32 or all bf16. Returns y (fp32).
    With delta_softplus, delta holds pre-activation values and the scan uses
    softplus(delta + delta_bias[d]) (delta_bias: (d,) fp32 or None)."""
    import torch
    lib = load_library()
    if direction not in DIRECTIONS:
        raise ValueError(f"direction must be one of {tuple(DIRECTIONS)}")
    dt = u.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("u must be float32 or bfloat16")
    for name, t in (("u", u), ("delta", delta), ("B", B), ("C", C)):
        _dev_tensor(t, name, (dt,))
    _dev_tensor(A, "A", (torch.float32,))
    _dev_tensor(D, "D", (torch.float32,))
    if u.dim() != 3 or A.dim() != 2 or B.dim() != 3:
        raise ValueError("expected u (batch, L, d), A (d, N), B/C (batch, L, N)")
    batch, L, d = u.shape
    N = A.shape[1]
    if delta.shape != u.shape or A.shape[0] != d or B.shape != (batch, L, N) \
            or C.shape != (batch, L, N) or D.shape != (d,):
        raise ValueError("inconsistent S6 shapes")
    if out is None:
        out = torch.empty(u.shape, dtype=torch.float32, device=u.device)
    else:
        _dev_tensor(out, "out", (torch.float32,))
        if out.shape != u.shape:
            raise ValueError("out must have u's shape")
    if delta_bias is not None:
        _dev_tensor(delta_bias, "delta_bias", (torch.float32,))
        if delta_bias.shape != (d,):
            raise ValueError("delta_bias must have shape (d,)")
    _same_device(u=u, delta=delta, A=A, B=B, C=C, D=D, delta_bias=delta_bias, out=out)
    if delta_softplus or delta_bias is not None:
        flags = (SSM_FLAG_BF16 if dt == torch.bfloat16 else 0) | \
            (SSM_FLAG_DELTA_SOFTPLUS if delta_softplus else 0)
        with torch.cuda.device(u.device):
            _check(lib.ssm_selective_scan_fwd_ex(
                u.data_ptr(), delta.data_ptr(),
                None if delta_bias is None else delta_bias.data_ptr(), A.data_ptr(),
                B.data_ptr(), C.data_ptr(), D.data_ptr(), out.data_ptr(), batch, L, d, N,
                DIRECTIONS[direction], flags, _stream(u)))
        return out
    fn = lib.ssm_selective_scan_fwd if dt == torch.float32 else lib.ssm_selective_scan_fwd_bf16
    with torch.cuda.device(u.device):
        _check(fn(u.data_ptr(), delta.data_ptr(), A.data_ptr(), B.data_ptr(), C.data_ptr(),
                  D.data_ptr(), out.data_ptr(), batch, L, d, N, DIRECTIONS[direction],
                  _stream(u)))
    return out


def copy_f32(src, dst):
    """dst[:] = src (fp32 device tensors of equal size), on the library's copy kernel."""
    import torch
    lib = load_library()
    _dev_tensor(src, "src", (torch.float32,))
    _dev_tensor(dst, "dst", (torch.float32,))
    if src.numel() != dst.numel():
        raise ValueError("src and dst sizes differ")
    _same_device(src=src, out_dst=dst)
    with torch.cuda.device(src.device):
        _check(lib.ssm_copy_f32(src.data_ptr(), dst.data_ptr(), src.numel(), _stream(src)))
    return dst


def stream_mul_f32(a, b, out=None):
    """out[:] = a * b (fp32 device tensors of equal size): the linear scan's
    traffic without the recurrence, on the library's stream kernel."""
    import torch
    lib = load_library()
    _dev_tensor(a, "a", (torch.float32,))
    _dev_tensor(b, "b", (torch.float32,))
    if a.numel() != b.numel():
        raise ValueError("a and b sizes differ")
    if out is None:
        out = torch.empty_like(a)
    _dev_tensor(out, "out", (torch.float32,))
    if out.numel() != a.numel():
        raise ValueError("out size differs from a")
    _same_device(a=a, b=b, out=out)
    with torch.cuda.device(a.device):
        _check(lib.ssm_stream_mul_f32(a.data_ptr(), b.data_ptr(), out.data_ptr(), a.numel(),
                                      _stream(a)))
    return out


def release_workspace():
    _check(load_library().ssm_release_workspace())
