// Single-pass decoupled look-back scan of the affine recurrence
//   h[t] = a[t] * h[t-1] + b[t],  h[-1] = h0
// for gfx950 (CDNA4, wave64).
//
// The recurrence is a prefix scan over affine maps m_t = (a_t, b_t) with the
// non-commutative composition (a1, b1) (+) (a2, b2) = (a1*a2, a2*b1 + b2),
// earlier map on the left ("Selective-scan CUDA kernels", the paragraph on the
// recurrence). The page's fastest design is a single-pass decoupled look-back
// with several items per thread scanned in registers and a warp-wide
// inspection of predecessors; this kernel keeps that structure and re-plans it
// for wave64, DPP and the multi-XCD memory system:
//
//  * tile = 4 waves x 4 rows x 64 lanes x float4 = 4096 elements. Each row is
//    read and written with one fully coalesced 1 KiB global_load/store_dwordx4
//    per wave, so no LDS transpose is needed.
//  * per lane: 4-element chunk aggregates in registers; per row: a wave64
//    inclusive scan of chunk aggregates with DPP row_shr / row_bcast steps;
//    per wave and per tile: short serial folds of 4 values.
//  * tile order comes from an atomic ticket, so every predecessor of a running
//    tile is itself running and will publish: forward progress holds.
//  * the status of a tile is three 64-bit words, each (epoch | fp32 payload),
//    written and read with relaxed agent-scope atomics. The payload is its own
//    flag, so there are no release/acquire fences (which would write back or
//    invalidate a whole L2 on this multi-XCD part) and no per-launch reset.
//  * look-back: wave 0 reads 64 predecessors per step (lane i -> tile k-1-i),
//    ballots for the nearest one whose inclusive value is published, and then
//    folds the aggregates in between strictly left to right, one lane at a
//    time. Every tile's inclusive value is therefore the same left fold
//    inc(k) = fma(G_k.a, inc(k-1), G_k.b) whichever predecessor was found,
//    which makes the output bitwise identical from run to run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace ssm {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowElems = 256;                    // 64 lanes x float4
constexpr int kWaveElems = kRowElems * kRows;     // 1024
constexpr int kTileElems = kWaveElems * kWaves;   // 4096

// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

template <int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ float dpp(float old, float src) {
  // Lanes whose source is out of the row/wave, or that are masked off, keep `old`.
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(old), __float_as_int(src), Ctrl, RowMask, BankMask, false));
}

// One Hillis-Steele step: (a, b) <- (a', b') (+) (a, b) where (a', b') comes
// from the lane the DPP control selects; lanes with no such lane combine with
// the identity (1, 0).
template <int Ctrl, int RowMask, int BankMask>
__device__ __forceinline__ void scan_step(float &a, float &b) {
  const float pa = dpp<Ctrl, RowMask, BankMask>(1.0f, a);
  const float pb = dpp<Ctrl, RowMask, BankMask>(0.0f, b);
  b = __builtin_fmaf(a, pb, b);
  a = pa * a;
}

// Inclusive wave64 scan of affine pairs in lane order (lane 0 earliest).
__device__ __forceinline__ void wave_scan(float &a, float &b) {
  scan_step<kRowShr1, 0xf, 0xf>(a, b);
  scan_step<kRowShr2, 0xf, 0xf>(a, b);
  scan_step<kRowShr4, 0xf, 0xf>(a, b);
  scan_step<kRowShr8, 0xf, 0xf>(a, b);
  scan_step<kRowBcast15, 0xa, 0xf>(a, b);   // rows 1, 3 take row 0, 2 totals
  scan_step<kRowBcast31, 0xc, 0xf>(a, b);   // rows 2, 3 take rows 0-1 total
}

__device__ __forceinline__ float lane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ uint64_t ld_status(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint64_t *p, uint32_t epoch, float v) {
  const uint64_t w = (uint64_t(epoch) << 32) | uint64_t(__float_as_uint(v));
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float payload(uint64_t w) {
  return __uint_as_float(uint32_t(w));
}

// h value entering tile `tile` (> 0): nearest published inclusive value of a
// predecessor, then the aggregates after it folded one by one, oldest first.
// Called by all 64 lanes of one wave; returns the same value in every lane.
__device__ float look_back(const TileStatus *st, int64_t tile, uint32_t epoch, int lane) {
  int64_t base = tile - 1;  // lane 0 inspects `base`, lane i inspects base - i
  int skipped = 0;          // whole windows of aggregates passed over so far
  for (;;) {
    const int64_t idx = base - lane;
    const bool valid = idx >= 0;
    uint64_t wi = 0, wa = 0, wb = 0;
    if (valid) {
      wi = ld_status(&st[idx].inc);
      wa = ld_status(&st[idx].agg_a);
      wb = ld_status(&st[idx].agg_b);
    }
    const bool is_inc = valid && uint32_t(wi >> 32) == epoch;
    const bool is_agg = valid && uint32_t(wa >> 32) == epoch && uint32_t(wb >> 32) == epoch;
    const uint64_t inc_mask = __ballot(is_inc);
    const uint64_t agg_mask = __ballot(is_agg);
    if (inc_mask != 0) {
      const int p = __builtin_ctzll(inc_mask);
      const uint64_t nearer = (p == 0) ? 0ull : ((1ull << p) - 1ull);
      if ((agg_mask & nearer) == nearer) {
        const float fa = payload(wa), fb = payload(wb);
        float h = lane_f(payload(wi), p);
        for (int l = p - 1; l >= 0; --l) h = __builtin_fmaf(lane_f(fa, l), h, lane_f(fb, l));
        // Windows passed over earlier are newer than this one: fold them in,
        // oldest (largest lane, farthest window) first. They are all complete.
        for (int w = 1; w <= skipped; ++w) {
          const int64_t j = base + 64 * w - lane;
          const float ga = payload(ld_status(&st[j].agg_a));
          const float gb = payload(ld_status(&st[j].agg_b));
          for (int l = 63; l >= 0; --l) h = __builtin_fmaf(lane_f(ga, l), h, lane_f(gb, l));
        }
        return h;
      }
    } else if ((agg_mask | ~__ballot(valid)) == ~0ull) {
      base -= 64;  // a full window of aggregates and no inclusive: look further back
      ++skipped;
      continue;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__global__ __launch_bounds__(kThreads) void linear_scan_kernel(
    const float *__restrict__ a, const float *__restrict__ b, float h0,
    float *__restrict__ h, int64_t n, int64_t ntiles, TileStatus *__restrict__ st,
    unsigned long long *__restrict__ ticket, unsigned long long ticket_base,
    uint32_t epoch) {
  __shared__ int64_t s_tile;
  __shared__ float s_wave_a[kWaves], s_wave_b[kWaves], s_carry[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  if (tid == 0) {
    const unsigned long long t =
        __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_tile = int64_t(t - ticket_base);
  }
  __syncthreads();
  const int64_t tile = s_tile;
  if (tile < 0 || tile >= ntiles) return;  // stale ticket base: never touch memory

  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  const bool full = (tile + 1) * kTileElems <= n;

  float4 va[kRows], vb[kRows];
  if (full) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t off = wave_start + r * kRowElems + lane * 4;
      va[r] = *reinterpret_cast<const float4 *>(a + off);
      vb[r] = *reinterpret_cast<const float4 *>(b + off);
    }
  } else {
    // Ragged last tile: elements past n are the identity map (1, 0).
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t off = wave_start + r * kRowElems + lane * 4;
      float ta[4], tb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = off + j < n;
        ta[j] = in ? a[off + j] : 1.0f;
        tb[j] = in ? b[off + j] : 0.0f;
      }
      va[r] = make_float4(ta[0], ta[1], ta[2], ta[3]);
      vb[r] = make_float4(tb[0], tb[1], tb[2], tb[3]);
    }
  }

  // Chunk aggregate of the lane's 4 items in each row, then a wave scan per row.
  float ia[kRows], ib[kRows];  // inclusive prefix of chunk aggregates within the row
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float ca = va[r].x, cb = vb[r].x;
    cb = __builtin_fmaf(va[r].y, cb, vb[r].y); ca *= va[r].y;
    cb = __builtin_fmaf(va[r].z, cb, vb[r].z); ca *= va[r].z;
    cb = __builtin_fmaf(va[r].w, cb, vb[r].w); ca *= va[r].w;
    wave_scan(ca, cb);
    ia[r] = ca;
    ib[r] = cb;
  }
  // Wave aggregate: rows folded in order.
  float wa = lane_f(ia[0], 63), wb = lane_f(ib[0], 63);
#pragma unroll
  for (int r = 1; r < kRows; ++r) {
    const float ra = lane_f(ia[r], 63), rb = lane_f(ib[r], 63);
    wb = __builtin_fmaf(ra, wb, rb);
    wa *= ra;
  }
  if (lane == 0) {
    s_wave_a[wave] = wa;
    s_wave_b[wave] = wb;
  }
  __syncthreads();

  if (wave == 0) {
    float ga = s_wave_a[0], gb = s_wave_b[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      gb = __builtin_fmaf(s_wave_a[w], gb, s_wave_b[w]);
      ga *= s_wave_a[w];
    }
    float h_in;
    if (tile == 0) {
      h_in = h0;
    } else {
      if (lane == 0) {
        st_status(&st[tile].agg_a, epoch, ga);
        st_status(&st[tile].agg_b, epoch, gb);
      }
      h_in = look_back(st, tile, epoch, lane);
    }
    if (lane == 0) {
      st_status(&st[tile].inc, epoch, __builtin_fmaf(ga, h_in, gb));
      float c = h_in;
      for (int w = 0; w < kWaves; ++w) {
        s_carry[w] = c;
        c = __builtin_fmaf(s_wave_a[w], c, s_wave_b[w]);
      }
    }
  }
  __syncthreads();

  // Apply: carry into each row, then into each lane's chunk, then re-run the
  // recurrence over the lane's 4 items.
  float c = s_carry[wave];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const float end = __builtin_fmaf(ia[r], c, ib[r]);      // h after this lane's chunk
    const float cin = dpp<kWaveShr1, 0xf, 0xf>(c, end);     // h before it
    float4 o;
    o.x = __builtin_fmaf(va[r].x, cin, vb[r].x);
    o.y = __builtin_fmaf(va[r].y, o.x, vb[r].y);
    o.z = __builtin_fmaf(va[r].z, o.y, vb[r].z);
    o.w = __builtin_fmaf(va[r].w, o.z, vb[r].w);
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    if (full) {
      *reinterpret_cast<float4 *>(h + off) = o;
    } else {
      const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (off + j < n) h[off + j] = ov[j];
    }
    c = lane_f(end, 63);
  }
}

__global__ __launch_bounds__(256) void copy_kernel(const float *__restrict__ src,
                                                   float *__restrict__ dst, int64_t n) {
  const int64_t nvec = n / 4;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nvec; i += stride)
    reinterpret_cast<float4 *>(dst)[i] = reinterpret_cast<const float4 *>(src)[i];
  for (int64_t i = nvec * 4 + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

int64_t linear_tile_elems() { return kTileElems; }

hipError_t launch_linear_scan(const float *a, const float *b, float h0, float *h,
                              int64_t n, int64_t ntiles, TileStatus *status,
                              unsigned long long *ticket,
                              unsigned long long ticket_base, uint32_t epoch,
                              hipStream_t stream) {
  hipLaunchKernelGGL(linear_scan_kernel, dim3(unsigned(ntiles)), dim3(kThreads), 0, stream,
                     a, b, h0, h, n, ntiles, status, ticket, ticket_base, epoch);
  return hipGetLastError();
}

hipError_t launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream) {
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

}  // namespace ssm
