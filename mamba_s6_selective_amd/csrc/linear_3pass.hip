// Three-pass scan of the affine recurrence h[t] = a[t]*h[t-1] + b[t],
// h[-1] = h0 ("Selective-scan CUDA kernels": the three-pass multi-block
// version that the page's memory-traffic model compares the single-pass
// look-back against).
//
//  1. local pass: each tile of 8192 elements composes its maps in order and
//     writes, for every element, the composition (A, B) of the tile's maps up
//     to and including it (8 B read, 8 B written per element), plus the
//     tile's aggregate;
//  2. carry pass: one workgroup folds the tile aggregates left to right and
//     writes the value of h entering every tile;
//  3. apply pass: h = A * h_in(tile) + B (8 B read, 4 B written per element).
//
// 28 B of HBM traffic per element against the single pass's 12 (read a, b;
// write h): the traffic model predicts the single pass 28/12 = 2.33x faster
// when both run at the same fraction of the bandwidth. The passes use the same
// composition rule and fixed shapes, so the result is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "scan_common.h"

namespace ssm {
namespace {

using namespace scan;

constexpr int kWaves = 4;
constexpr int kRows = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowElems = 256;                   // 64 lanes x float4
constexpr int kWaveElems = kRowElems * kRows;    // 2048
constexpr int kTileElems = kWaveElems * kWaves;  // 8192

// Composition (x (+) y), x earlier.
__device__ __forceinline__ void compose(float xa, float xb, float ya, float yb, float &ra,
                                        float &rb) {
  rb = __builtin_fmaf(ya, xb, yb);
  ra = xa * ya;
}

__global__ __launch_bounds__(kThreads) void local_kernel(const float *__restrict__ a,
                                                         const float *__restrict__ b,
                                                         float *__restrict__ pa,
                                                         float *__restrict__ pb,
                                                         float *__restrict__ agg, int64_t n) {
  __shared__ float s_wa[kWaves], s_wb[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  const bool full = (tile + 1) * kTileElems <= n;
  float4 va[kRows], vb[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    if (full) {
      va[r] = load_nt(a + off);
      vb[r] = load_nt(b + off);
    } else {  // past n: the identity map (1, 0)
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
  // Per row: the lanes' exclusive prefixes within the row; the rows' prefixes
  // within the wave (serial); the wave's total.
  float ea[kRows], eb[kRows];
  float ra = 1.0f, rb = 0.0f;  // composition of the wave's earlier rows
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float ca = va[r].x, cb = vb[r].x;
    compose(ca, cb, va[r].y, vb[r].y, ca, cb);
    compose(ca, cb, va[r].z, vb[r].z, ca, cb);
    compose(ca, cb, va[r].w, vb[r].w, ca, cb);
    wave_scan(ca, cb);
    const float xa = dpp<kWaveShr1, 0xf, 0xf>(1.0f, ca);  // lanes before this one
    const float xb = dpp<kWaveShr1, 0xf, 0xf>(0.0f, cb);
    compose(ra, rb, xa, xb, ea[r], eb[r]);
    compose(ra, rb, lane_f(ca, 63), lane_f(cb, 63), ra, rb);
  }
  if (lane == 0) {
    s_wa[wave] = ra;
    s_wb[wave] = rb;
  }
  __syncthreads();
  float wa = 1.0f, wb = 0.0f;  // composition of the tile's earlier waves
  for (int w = 0; w < wave; ++w) compose(wa, wb, s_wa[w], s_wb[w], wa, wb);
  if (wave == kWaves - 1 && lane == 0) {
    float ta, tb;
    compose(wa, wb, ra, rb, ta, tb);
    agg[2 * tile] = ta;
    agg[2 * tile + 1] = tb;
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float qa, qb;
    compose(wa, wb, ea[r], eb[r], qa, qb);  // everything before the lane's first item
    float4 oa, ob;
    compose(qa, qb, va[r].x, vb[r].x, oa.x, ob.x);
    compose(oa.x, ob.x, va[r].y, vb[r].y, oa.y, ob.y);
    compose(oa.y, ob.y, va[r].z, vb[r].z, oa.z, ob.z);
    compose(oa.z, ob.z, va[r].w, vb[r].w, oa.w, ob.w);
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    if (full) {
      store_nt(pa + off, oa);
      store_nt(pb + off, ob);
    } else {
      const float xa4[4] = {oa.x, oa.y, oa.z, oa.w}, xb4[4] = {ob.x, ob.y, ob.z, ob.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (off + j < n) {
          pa[off + j] = xa4[j];
          pb[off + j] = xb4[j];
        }
    }
  }
}

// Local pass by a register-resident Hillis-Steele scan ("Selective-scan CUDA
// kernels" measured Hillis-Steele only as a PyTorch version and called the
// comparison with its kernels not yet fair for that reason). Each row of 256
// elements (64 lanes x 4 in registers) is scanned in log2(256) = 8 steps; in
// the step of distance d every element e >= d becomes old[e-d] (+) old[e],
// all reads taking the values from before the step: O(n log n) compositions
// instead of the work-efficient pass's O(n). Neighbouring lanes' values come
// through cross-lane shuffles. Rows, waves and the tile then combine as in
// local_kernel, and the output is the same (A, B) per element.
__device__ __forceinline__ float shfl_up_f(float v, int s) { return __shfl_up(v, s); }

__device__ __forceinline__ void hs_row(float (&A)[4], float (&B)[4], int lane) {
  float nA[4], nB[4];
  {  // d = 1: element 4l+j reads 4l+j-1; item 0 reads the previous lane's item 3
    const float pa = shfl_up_f(A[3], 1), pb = shfl_up_f(B[3], 1);
    if (lane >= 1) compose(pa, pb, A[0], B[0], nA[0], nB[0]); else { nA[0] = A[0]; nB[0] = B[0]; }
#pragma unroll
    for (int j = 1; j < 4; ++j) compose(A[j - 1], B[j - 1], A[j], B[j], nA[j], nB[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) { A[j] = nA[j]; B[j] = nB[j]; }
  }
  {  // d = 2: items 0, 1 read the previous lane's items 2, 3
    const float pa2 = shfl_up_f(A[2], 1), pb2 = shfl_up_f(B[2], 1);
    const float pa3 = shfl_up_f(A[3], 1), pb3 = shfl_up_f(B[3], 1);
    if (lane >= 1) {
      compose(pa2, pb2, A[0], B[0], nA[0], nB[0]);
      compose(pa3, pb3, A[1], B[1], nA[1], nB[1]);
    } else {
      nA[0] = A[0]; nB[0] = B[0]; nA[1] = A[1]; nB[1] = B[1];
    }
    compose(A[0], B[0], A[2], B[2], nA[2], nB[2]);
    compose(A[1], B[1], A[3], B[3], nA[3], nB[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) { A[j] = nA[j]; B[j] = nB[j]; }
  }
#pragma unroll
  for (int s = 1; s < 64; s *= 2) {  // d = 4s: the same item s lanes back
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pa = shfl_up_f(A[j], s), pb = shfl_up_f(B[j], s);
      if (lane >= s) compose(pa, pb, A[j], B[j], nA[j], nB[j]); else { nA[j] = A[j]; nB[j] = B[j]; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { A[j] = nA[j]; B[j] = nB[j]; }
  }
}

__global__ __launch_bounds__(kThreads) void local_hs_kernel(const float *__restrict__ a,
                                                            const float *__restrict__ b,
                                                            float *__restrict__ pa,
                                                            float *__restrict__ pb,
                                                            float *__restrict__ agg, int64_t n) {
  __shared__ float s_wa[kWaves], s_wb[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  const bool full = (tile + 1) * kTileElems <= n;
  float A[kRows][4], B[kRows][4];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    if (full) {
      const float4 x = load_nt(a + off), y = load_nt(b + off);
      A[r][0] = x.x; A[r][1] = x.y; A[r][2] = x.z; A[r][3] = x.w;
      B[r][0] = y.x; B[r][1] = y.y; B[r][2] = y.z; B[r][3] = y.w;
    } else {  // past n: the identity map (1, 0)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = off + j < n;
        A[r][j] = in ? a[off + j] : 1.0f;
        B[r][j] = in ? b[off + j] : 0.0f;
      }
    }
  }
  float ea[kRows], eb[kRows];  // composition of the wave's rows before row r
  float ra = 1.0f, rb = 0.0f;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    hs_row(A[r], B[r], lane);
    ea[r] = ra;
    eb[r] = rb;
    compose(ra, rb, lane_f(A[r][3], 63), lane_f(B[r][3], 63), ra, rb);
  }
  if (lane == 0) {
    s_wa[wave] = ra;
    s_wb[wave] = rb;
  }
  __syncthreads();
  float wa = 1.0f, wb = 0.0f;  // composition of the tile's earlier waves
  for (int w = 0; w < wave; ++w) compose(wa, wb, s_wa[w], s_wb[w], wa, wb);
  if (wave == kWaves - 1 && lane == 0) {
    float ta, tb;
    compose(wa, wb, ra, rb, ta, tb);
    agg[2 * tile] = ta;
    agg[2 * tile + 1] = tb;
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    float qa, qb;
    compose(wa, wb, ea[r], eb[r], qa, qb);  // everything before the row
    float oa[4], ob[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) compose(qa, qb, A[r][j], B[r][j], oa[j], ob[j]);
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    if (full) {
      store_nt(pa + off, make_float4(oa[0], oa[1], oa[2], oa[3]));
      store_nt(pb + off, make_float4(ob[0], ob[1], ob[2], ob[3]));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (off + j < n) {
          pa[off + j] = oa[j];
          pb[off + j] = ob[j];
        }
    }
  }
}

// One workgroup of kCarryWaves waves. Wave w owns rows [w*rows, (w+1)*rows)
// of 64 consecutive tile aggregates, lane l holding tile row*64 + l, so every
// load of a row and every store of its incoming values moves 64 neighbouring
// entries. First walk: each row is scanned across lanes (DPP) and the rows'
// totals are composed in order into the wave's total; the totals meet in LDS.
// Second walk: each wave goes over its rows again from the composition of the
// waves before it, writing the value of h entering each tile. Rows are read
// kBatch at a time, every load issued before any is used (and, up to kBatch
// rows per wave, the second walk reads no memory). Fixed shapes, so the
// result is deterministic.
constexpr int kCarryThreads = 1024;
constexpr int kCarryWaves = kCarryThreads / 64;
constexpr int kBatch = 16;

__global__ __launch_bounds__(kCarryThreads) void carry_kernel(const float *__restrict__ agg,
                                                              float *__restrict__ hin,
                                                              float h0, int64_t ntiles,
                                                              int64_t rows) {
  __shared__ float s_a[kCarryWaves], s_b[kCarryWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t first = int64_t(wave) * rows;  // the wave's first row
  float ia[kBatch], ib[kBatch];                // inclusive scans of a batch of rows
  // Rows k0 .. k0 + kBatch - 1 of the wave, each scanned across lanes; tiles
  // past the wave's rows or past the end are the identity.
  auto scan_batch = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t t = (first + k0 + j) * 64 + lane;
      const int64_t tc = t < ntiles ? t : ntiles - 1;
      ia[j] = agg[2 * tc];
      ib[j] = agg[2 * tc + 1];
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = k0 + j < rows && (first + k0 + j) * 64 + lane < ntiles;
      ia[j] = in ? ia[j] : 1.0f;
      ib[j] = in ? ib[j] : 0.0f;
      wave_scan(ia[j], ib[j]);
    }
  };
  float ta = 1.0f, tb = 0.0f;  // the wave's total, the same in every lane
  for (int64_t k0 = 0; k0 < rows; k0 += kBatch) {
    scan_batch(k0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) compose(ta, tb, lane_f(ia[j], 63), lane_f(ib[j], 63), ta, tb);
  }
  if (lane == 0) {
    s_a[wave] = ta;
    s_b[wave] = tb;
  }
  __syncthreads();
  float wa = 1.0f, wb = 0.0f;  // earlier waves
  for (int w = 0; w < wave; ++w) compose(wa, wb, s_a[w], s_b[w], wa, wb);
  float h = __builtin_fmaf(wa, h0, wb);  // entering the wave's first row
  const bool cached = rows <= kBatch;    // same for every wave
  for (int64_t k0 = 0; k0 < rows; k0 += kBatch) {
    if (!cached) scan_batch(k0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float xa = dpp<kWaveShr1, 0xf, 0xf>(1.0f, ia[j]);  // earlier lanes of the row
      const float xb = dpp<kWaveShr1, 0xf, 0xf>(0.0f, ib[j]);
      const int64_t t = (first + k0 + j) * 64 + lane;
      if (k0 + j < rows && t < ntiles) hin[t] = __builtin_fmaf(xa, h, xb);
      h = __builtin_fmaf(lane_f(ia[j], 63), h, lane_f(ib[j], 63));
    }
  }
}

// 1024 elements per workgroup (one float4 per thread); the tile's incoming
// value is wave-uniform.
__global__ __launch_bounds__(256) void apply_kernel(const float *__restrict__ pa,
                                                    const float *__restrict__ pb,
                                                    const float *__restrict__ hin,
                                                    float *__restrict__ h, int64_t n) {
  const int64_t off = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const float c = hin[(int64_t(blockIdx.x) * 1024) / kTileElems];
  if (off + 4 <= n) {
    const float4 A = load_nt(pa + off), B = load_nt(pb + off);
    float4 o;
    o.x = __builtin_fmaf(A.x, c, B.x);
    o.y = __builtin_fmaf(A.y, c, B.y);
    o.z = __builtin_fmaf(A.z, c, B.z);
    o.w = __builtin_fmaf(A.w, c, B.w);
    store_nt(h + off, o);
  } else {
    for (int64_t i = off; i < n; ++i) h[i] = __builtin_fmaf(pa[i], c, pb[i]);
  }
}

}  // namespace

int64_t linear3_tile_elems() { return kTileElems; }

size_t linear3_workspace_bytes(int64_t n) {
  const int64_t ntiles = (n + kTileElems - 1) / kTileElems;
  const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(size_t(n) * 4) * 2 + up(size_t(ntiles) * 8) + up(size_t(ntiles) * 4);
}

hipError_t launch_linear_scan_3pass(const float *a, const float *b, float h0, float *h,
                                    int64_t n, void *workspace, bool hillis_steele,
                                    hipStream_t stream) {
  const int64_t ntiles = (n + kTileElems - 1) / kTileElems;
  const auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char *w = static_cast<char *>(workspace);
  float *pa = reinterpret_cast<float *>(w);
  float *pb = reinterpret_cast<float *>(w + up(size_t(n) * 4));
  float *agg = reinterpret_cast<float *>(w + 2 * up(size_t(n) * 4));
  float *hin = reinterpret_cast<float *>(w + 2 * up(size_t(n) * 4) + up(size_t(ntiles) * 8));
  if (hillis_steele)
    hipLaunchKernelGGL(local_hs_kernel, dim3(unsigned(ntiles)), dim3(kThreads), 0, stream, a, b,
                       pa, pb, agg, n);
  else
    hipLaunchKernelGGL(local_kernel, dim3(unsigned(ntiles)), dim3(kThreads), 0, stream, a, b, pa,
                       pb, agg, n);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t rows = (ntiles + kCarryThreads - 1) / kCarryThreads;  // per wave, of 64 tiles
  hipLaunchKernelGGL(carry_kernel, dim3(1), dim3(kCarryThreads), 0, stream, agg, hin, h0, ntiles,
                     rows);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t groups = (n + 1023) / 1024;
  hipLaunchKernelGGL(apply_kernel, dim3(unsigned(groups)), dim3(256), 0, stream, pa, pb, hin, h,
                     n);
  return hipGetLastError();
}

}  // namespace ssm
