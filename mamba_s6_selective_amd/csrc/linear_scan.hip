// Single-pass look-back scan of the affine recurrence
//   h[t] = a[t] * h[t-1] + b[t],  h[-1] = h0
// for gfx950 (CDNA4, wave64).
//
// The recurrence is a prefix scan over affine maps m_t = (a_t, b_t) with the
// non-commutative composition (a1, b1) (+) (a2, b2) = (a1*a2, a2*b1 + b2),
// earlier map on the left ("Selective-scan CUDA kernels", the paragraph on the
// recurrence). The page's fastest design is a single-pass decoupled look-back
// with several items per thread scanned in registers and a warp-wide
// inspection of predecessors. This kernel keeps the single pass, the
// register-resident items and the wave-wide inspection, and re-plans the
// cross-tile protocol for a part whose workgroups sit on 8 XCDs with private
// L2s, where a published word takes on the order of a microsecond to become
// visible to another XCD:
//
//  * tile = 4 waves x 8 rows x 64 lanes x float4 = 8192 elements. Each row is
//    read and written with one fully coalesced 1 KiB global_load/store_dwordx4
//    per wave (no LDS transpose). Per lane: 4-element chunk aggregates in
//    registers; per row: a wave64 inclusive scan of chunk aggregates with DPP
//    row_shr / row_bcast steps; per wave and per tile: short serial folds.
//  * no inclusive-prefix chain. A classic look-back publishes each tile's
//    inclusive prefix, and the published frontier then advances by at most
//    one inspection window per visibility round trip. Here every tile only
//    publishes aggregates, at three levels: its own (level 0), that of its
//    superblock of 64 tiles (level 1, published by the superblock's last
//    tile), and that of its block of 64 superblocks (level 2, published by
//    the block's last tile). A tile's incoming value is h0 pushed through the
//    composition of at most 63 level-2, 63 level-1 and 63 level-0 aggregates,
//    each window composed by one fixed-shape wave64 DPP scan. Every wait is on
//    aggregates that depend only on loads of earlier tiles, so a tile waits a
//    bounded number of round trips, whatever the size of the input.
//  * deterministic: the window contents and the shape of every composition are
//    fixed by the tile index alone, so the output is bitwise identical from
//    run to run.
//  * status words are 64-bit (epoch | fp32 payload), written and read with
//    relaxed agent-scope atomics. The payload is its own flag, so there are no
//    release/acquire fences (which would write back or invalidate a whole L2)
//    and no per-launch reset.
//  * the kernel is persistent and launched cooperatively: every workgroup is
//    resident and walks its tiles in increasing order, and a tile only waits
//    for words published by lower tiles before they wait on anything, so the
//    lowest unfinished tile can always finish.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace ssm {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowElems = 256;                    // 64 lanes x float4
constexpr int kWaveElems = kRowElems * kRows;     // 2048
constexpr int kTileElems = kWaveElems * kWaves;   // 8192
constexpr int kFan = 64;                          // entries per look-back window

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

__device__ __forceinline__ bool word_ready(uint64_t w, uint32_t epoch) {
  return uint32_t(w >> 32) == epoch;
}

// Composition, in lane order, of the pairs held by lanes [0, count) of the
// wave (later lanes contribute the identity). Fixed DPP tree: the result
// depends only on the values and `count`. Returned in every lane.
__device__ __forceinline__ void window_total(float a, float b, int count, int lane, float &ta,
                                             float &tb) {
  if (lane >= count) {
    a = 1.0f;
    b = 0.0f;
  }
  wave_scan(a, b);
  ta = lane_f(a, 63);
  tb = lane_f(b, 63);
}

// Incoming value of `tile`, composed from published aggregates (see the file
// comment). The last tile of a superblock also publishes the superblock's
// aggregate, and the last tile of a block the block's aggregate, as soon as
// their inputs are visible. Called by all 64 lanes of one wave.
__device__ float look_back(const LinearStatus &st, int64_t tile, float ga, float gb, float h0,
                           uint32_t epoch, int lane) {
  const int64_t sb = tile / kFan;             // superblock of this tile
  const int64_t blk = sb / kFan;              // block of this tile
  const int n0 = int(tile - sb * kFan);       // level-0 entries before the tile in its superblock
  const int n1 = int(sb - blk * kFan);        // level-1 entries before its superblock in its block
  const int n2 = int(blk);                    // level-2 entries before its block
  const bool last_in_sb = n0 == kFan - 1;
  const bool last_in_blk = last_in_sb && n1 == kFan - 1;
  const bool need0 = lane < n0, need1 = lane < n1, need2 = lane < n2;
  const int64_t i0 = sb * kFan + lane, i1 = blk * kFan + lane, i2 = lane;
  uint64_t w0a = 0, w0b = 0, w1a = 0, w1b = 0, w2a = 0, w2b = 0;
  bool r0 = !need0, r1 = !need1, r2 = !need2;
  bool pub1 = !last_in_sb, pub2 = !last_in_blk;
  float sa = 1.0f, sbv = 0.0f;  // this superblock's aggregate, when published here
  for (;;) {
    if (!r0) {
      w0a = ld_status(&st.lvl0[i0].a);
      w0b = ld_status(&st.lvl0[i0].b);
      r0 = word_ready(w0a, epoch) && word_ready(w0b, epoch);
    }
    if (!r1) {
      w1a = ld_status(&st.lvl1[i1].a);
      w1b = ld_status(&st.lvl1[i1].b);
      r1 = word_ready(w1a, epoch) && word_ready(w1b, epoch);
    }
    if (!r2) {
      w2a = ld_status(&st.lvl2[i2].a);
      w2b = ld_status(&st.lvl2[i2].b);
      r2 = word_ready(w2a, epoch) && word_ready(w2b, epoch);
    }
    const bool all0 = __ballot(!r0) == 0, all1 = __ballot(!r1) == 0, all2 = __ballot(!r2) == 0;
    if (!pub1 && all0) {
      float pa, pb;
      window_total(payload(w0a), payload(w0b), n0, lane, pa, pb);
      sbv = __builtin_fmaf(ga, pb, gb);  // (P0 (+) own aggregate)
      sa = pa * ga;
      if (lane == 0) {
        st_status(&st.lvl1[sb].a, epoch, sa);
        st_status(&st.lvl1[sb].b, epoch, sbv);
      }
      pub1 = true;
    }
    if (!pub2 && pub1 && all1) {
      float pa, pb;
      window_total(payload(w1a), payload(w1b), n1, lane, pa, pb);
      if (lane == 0) {
        st_status(&st.lvl2[blk].a, epoch, pa * sa);
        st_status(&st.lvl2[blk].b, epoch, __builtin_fmaf(sa, pb, sbv));
      }
      pub2 = true;
    }
    if (all0 && all1 && all2 && pub1 && pub2) break;
    __builtin_amdgcn_s_sleep(1);
  }
  float p0a, p0b, p1a, p1b, p2a, p2b;
  window_total(payload(w0a), payload(w0b), n0, lane, p0a, p0b);
  window_total(payload(w1a), payload(w1b), n1, lane, p1a, p1b);
  window_total(payload(w2a), payload(w2b), n2, lane, p2a, p2b);
  const float h2 = __builtin_fmaf(p2a, h0, p2b);
  const float h1 = __builtin_fmaf(p1a, h2, p1b);
  return __builtin_fmaf(p0a, h1, p0b);
}

// One tile: load, scan in registers, publish, look back, apply, store.
__device__ __forceinline__ void scan_tile(const float *__restrict__ a,
                                          const float *__restrict__ b, float h0,
                                          float *__restrict__ h, int64_t n, int64_t tile,
                                          const LinearStatus &st, uint32_t epoch,
                                          float *s_wave_a, float *s_wave_b, float *s_carry) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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
    if (lane == 0) {
      st_status(&st.lvl0[tile].a, epoch, ga);
      st_status(&st.lvl0[tile].b, epoch, gb);
    }
    const float h_in = look_back(st, tile, ga, gb, h0, epoch, lane);
    if (lane == 0) {
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

// Persistent kernel: launched cooperatively, so all gridDim.x workgroups are
// resident at once. Workgroup w scans tiles w, w + G, w + 2G, ... in order.
// A tile only waits for lower-numbered tiles, each of which belongs to a
// resident workgroup that reaches it after finishing its own lower tiles;
// the lowest unfinished tile can therefore always finish (no ticket needed).
__global__ __launch_bounds__(kThreads) void linear_scan_kernel(
    const float *__restrict__ a, const float *__restrict__ b, float h0,
    float *__restrict__ h, int64_t n, int64_t ntiles, LinearStatus st, uint32_t epoch) {
  __shared__ float s_wave_a[kWaves], s_wave_b[kWaves], s_carry[kWaves];
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    scan_tile(a, b, h0, h, n, tile, st, epoch, s_wave_a, s_wave_b, s_carry);
    __syncthreads();  // s_carry is rewritten by the next tile
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
                              int64_t n, int64_t ntiles, LinearStatus status, uint32_t epoch,
                              int resident_wgs, hipStream_t stream) {
  const unsigned grid = unsigned(ntiles < resident_wgs ? ntiles : resident_wgs);
  void *args[] = {(void *)&a, (void *)&b, (void *)&h0, (void *)&h,
                  (void *)&n, (void *)&ntiles, (void *)&status, (void *)&epoch};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(linear_scan_kernel),
                                    dim3(grid), dim3(kThreads), args, 0, stream);
}

int linear_wgs_per_cu() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(linear_scan_kernel), kThreads, 0) !=
      hipSuccess)
    return 0;
  return per_cu;
}

hipError_t launch_copy_f32(const float *src, float *dst, int64_t n, hipStream_t stream) {
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, src, dst, n);
  return hipGetLastError();
}

}  // namespace ssm
