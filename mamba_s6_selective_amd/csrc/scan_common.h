// Device helpers shared by the linear-recurrence scan kernels: wave64 DPP
// scans of affine pairs and streaming 16-byte loads/stores (gfx950).
//
// An affine pair (a, b) is the map h -> a*h + b; composition in sequence
// order is (a1, b1) (+) (a2, b2) = (a1*a2, a2*b1 + b2), earlier map on the
// left ("Selective-scan CUDA kernels", the paragraph on the recurrence).
#pragma once

#include <hip/hip_runtime.h>

namespace ssm {
namespace scan {

// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

template <int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ float dpp(float old, float src) {
  // Lanes whose source is out of the row/wave, or that are masked off, keep `old`.
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(old), __float_as_int(src), Ctrl, RowMask, BankMask, false));
}

// Composition rules for affine pairs. `apply` is the map (a, b) applied to a
// value h; `compose` is (x (+) y) with x earlier.
//  PlainOp - IEEE arithmetic throughout (a zero multiplier times an inf or
//            NaN state is NaN, as in the sequential loop).
//  ResetOp - a multiplier of exactly zero discards everything before it, an
//            inf or NaN included: a sequence boundary inside one scan is then
//            exact, and nothing of one sequence leaks into the next.
struct PlainOp {
  static __device__ __forceinline__ float apply(float a, float h, float b) {
    return __builtin_fmaf(a, h, b);
  }
  static __device__ __forceinline__ void compose(float xa, float xb, float ya, float yb,
                                                 float &ra, float &rb) {
    const float nb = __builtin_fmaf(ya, xb, yb);
    ra = xa * ya;
    rb = nb;
  }
};
struct ResetOp {
  static __device__ __forceinline__ float apply(float a, float h, float b) {
    return a == 0.0f ? b : __builtin_fmaf(a, h, b);
  }
  static __device__ __forceinline__ void compose(float xa, float xb, float ya, float yb,
                                                 float &ra, float &rb) {
    const bool cut = ya == 0.0f;
    const float nb = cut ? yb : __builtin_fmaf(ya, xb, yb);
    ra = cut ? 0.0f : xa * ya;
    rb = nb;
  }
};

// One Hillis-Steele step: (a, b) <- (a', b') (+) (a, b) where (a', b') comes
// from the lane the DPP control selects; lanes with no such lane combine with
// the identity (1, 0).
template <class Op, int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ void scan_step(float &a, float &b) {
  const float pa = dpp<Ctrl, RowMask, BankMask>(1.0f, a);
  const float pb = dpp<Ctrl, RowMask, BankMask>(0.0f, b);
  Op::compose(pa, pb, a, b, a, b);
}

// Inclusive wave64 scan of affine pairs in lane order (lane 0 earliest).
template <class Op = PlainOp>
__device__ __forceinline__ void wave_scan(float &a, float &b) {
  scan_step<Op, kRowShr1, 0xf, 0xf>(a, b);
  scan_step<Op, kRowShr2, 0xf, 0xf>(a, b);
  scan_step<Op, kRowShr4, 0xf, 0xf>(a, b);
  scan_step<Op, kRowShr8, 0xf, 0xf>(a, b);
  scan_step<Op, kRowBcast15, 0xa, 0xf>(a, b);   // rows 1, 3 take row 0, 2 totals
  scan_step<Op, kRowBcast31, 0xc, 0xf>(a, b);   // rows 2, 3 take rows 0-1 total
}

__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Streaming (non-temporal) 16-byte loads and stores, for data touched once
// that should not displace anything in L2 or the MALL.
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float *p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(float *p, float4 o) {
  const v4f v = {o.x, o.y, o.z, o.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(p));
}

}  // namespace scan
}  // namespace ssm
