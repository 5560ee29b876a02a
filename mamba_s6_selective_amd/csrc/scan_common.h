// Device helpers shared by the linear-recurrence scan kernels: affine maps and
// their composition rules, wave64 DPP scans of maps, and streaming 16-byte
// loads/stores (gfx950).
//
// An affine map (a, b) is h -> a*h + b; composition in sequence order is
// (a1, b1) (+) (a2, b2) = (a1*a2, a2*b1 + b2), earlier map on the left
// ("Selective-scan CUDA kernels", the paragraph on the recurrence).
//
// Non-finite values. The sequential loop h = a*h + b never multiplies two
// multipliers together; a scan does, and a product of many multipliers below
// one underflows to zero in fp32 although its exact value is not zero. A
// state of +-inf pushed through such a product would then give 0*inf = NaN
// where the loop keeps +-inf. So every multiplier a scan forms keeps "exactly
// zero" meaningful: a product of two non-zero factors that underflows is
// replaced by the smallest subnormal of its sign (mul_nz), which changes a
// finite result by at most 2^-149 times the state it multiplies, and turns
// inf into inf. Kernels take the careful rule everywhere a map with a
// non-finite part can meet an underflowed product, and a cheaper rule
// (underflowed zeros nudged after the fact) where all values are finite.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
template <int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ uint32_t dpp_u(uint32_t old, uint32_t src) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(old), int(src), Ctrl, RowMask, BankMask, false));
}

// An affine map h -> a*h + b. `head` is used by the batched scan only: it
// marks a map that holds the first element of a sequence, which ignores
// whatever comes before it (its b already holds that element's value).
struct Map {
  float a, b;
  uint32_t head;  // 0 or 1
};

__device__ __forceinline__ Map identity_map() { return Map{1.0f, 0.0f, 0u}; }

// The smallest subnormal with the sign of p, for p = +-0.
__device__ __forceinline__ float nudge(float p) { return __int_as_float(__float_as_int(p) | 1); }

// Multiplier of "x then y" with exact zeros kept meaningful: x == 0 gives x
// (a map with multiplier 0 is constant, and so is its composition with any
// later map, even one whose multiplier is inf or NaN: the loop never
// multiplies that zero by a later multiplier); otherwise the IEEE product,
// except that two non-zero factors whose product underflows give the smallest
// subnormal of the product's sign.
__device__ __forceinline__ float mul_nz(float x, float y) {
  const float p = x * y;
  const float q = (p == 0.0f && y != 0.0f) ? nudge(p) : p;
  return x == 0.0f ? x : q;
}

// A multiplier formed with plain products from factors that are all finite
// and non-zero: any zero is an underflow, so it is nudged.
__device__ __forceinline__ float fix_underflow(float p) { return p == 0.0f ? nudge(p) : p; }

// Composition rules. Seg: heads are honoured (batched scans). Careful: the
// multiplier product is mul_nz (needed wherever a non-finite value can meet
// an underflowed product); otherwise plain IEEE.
template <bool Seg, bool Careful>
struct AffOp {
  static constexpr bool kSeg = Seg;
  static __device__ __forceinline__ float apply(const Map &m, float h) {
    if constexpr (Seg) {
      if (m.head) return m.b;
    }
    return __builtin_fmaf(m.a, h, m.b);
  }
  // x earlier, y later.
  static __device__ __forceinline__ Map compose(const Map &x, const Map &y) {
    Map r;
    r.b = __builtin_fmaf(y.a, x.b, y.b);
    r.a = Careful ? mul_nz(x.a, y.a) : x.a * y.a;
    r.head = 0u;
    if constexpr (Seg) {
      r.head = x.head | y.head;
      if (y.head) {
        r.a = y.a;
        r.b = y.b;
      }
    }
    return r;
  }
};

// One Hillis-Steele step: m <- m' (+) m where m' comes from the lane the DPP
// control selects; lanes with no such lane combine with the identity.
template <class Op, int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ void scan_step(Map &m) {
  Map p;
  p.a = dpp<Ctrl, RowMask, BankMask>(1.0f, m.a);
  p.b = dpp<Ctrl, RowMask, BankMask>(0.0f, m.b);
  p.head = 0u;
  if constexpr (Op::kSeg) p.head = dpp_u<Ctrl, RowMask, BankMask>(0u, m.head);
  m = Op::compose(p, m);
}

// Inclusive wave64 scan of maps in lane order (lane 0 earliest).
template <class Op>
__device__ __forceinline__ void wave_scan(Map &m) {
  scan_step<Op, kRowShr1, 0xf, 0xf>(m);
  scan_step<Op, kRowShr2, 0xf, 0xf>(m);
  scan_step<Op, kRowShr4, 0xf, 0xf>(m);
  scan_step<Op, kRowShr8, 0xf, 0xf>(m);
  scan_step<Op, kRowBcast15, 0xa, 0xf>(m);   // rows 1, 3 take row 0, 2 totals
  scan_step<Op, kRowBcast31, 0xc, 0xf>(m);   // rows 2, 3 take rows 0-1 total
}

__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ Map lane_map(const Map &m, int lane) {
  return Map{lane_f(m.a, lane), lane_f(m.b, lane),
             uint32_t(__builtin_amdgcn_readlane(int(m.head), lane))};
}
// The map of the lane before this one (lane 0: the identity).
__device__ __forceinline__ Map prev_lane_map(const Map &m) {
  Map p;
  p.a = dpp<kWaveShr1, 0xf, 0xf>(1.0f, m.a);
  p.b = dpp<kWaveShr1, 0xf, 0xf>(0.0f, m.b);
  p.head = dpp_u<kWaveShr1, 0xf, 0xf>(0u, m.head);
  return p;
}

// Whether a wave-uniform value (an SGPR after readlane) is inf or NaN.
__device__ __forceinline__ bool uniform_nonfinite(float v) {
  return (__float_as_uint(v) & 0x7f800000u) == 0x7f800000u;
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
