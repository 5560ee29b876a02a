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

using COp = AffOp<false, true>;   // mul_nz products
using FOp = AffOp<false, false>;  // plain products

// Loads the wave's rows of one tile; past n the identity map (1, 0). Returns
// whether the wave may take the fast path: every a and b finite and no a
// exactly zero, so that a zero product of multipliers can only be an
// underflow (nudged), and no inf or NaN can meet one.
__device__ __forceinline__ bool load_rows(const float *__restrict__ a,
                                          const float *__restrict__ b, int64_t n,
                                          int64_t wave_start, float (&A)[kRows][4],
                                          float (&B)[kRows][4]) {
  const int lane = threadIdx.x & 63;
  const bool full = wave_start + kWaveElems <= n;
  bool odd = false;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    if (full) {
      const float4 x = load_nt(a + off), y = load_nt(b + off);
      A[r][0] = x.x; A[r][1] = x.y; A[r][2] = x.z; A[r][3] = x.w;
      B[r][0] = y.x; B[r][1] = y.y; B[r][2] = y.z; B[r][3] = y.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = off + j < n;
        A[r][j] = in ? a[off + j] : 1.0f;
        B[r][j] = in ? b[off + j] : 0.0f;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      // classes: NaN, +-inf and +-0 for a; NaN and +-inf for b
      odd = odd || __builtin_amdgcn_class(A[r][j], 0x267) || __builtin_amdgcn_class(B[r][j], 0x207);
  return __builtin_amdgcn_ballot_w64(odd) == 0;
}

// Stores the wave's rows of (A, B) pairs.
__device__ __forceinline__ void store_rows(float *__restrict__ pa, float *__restrict__ pb,
                                           int64_t n, int64_t wave_start, int r,
                                           const float (&oa)[4], const float (&ob)[4]) {
  const int lane = threadIdx.x & 63;
  const int64_t off = wave_start + r * kRowElems + lane * 4;
  if (off + 4 <= n) {
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

// Per row: the lanes' exclusive prefixes within the row; the rows' prefixes
// within the wave (serial); the wave's total. Fast (Careful == false): plain
// products, every zero multiplier nudged (only underflows can be zero).
template <bool Careful>
__device__ __forceinline__ Map rows_prefix(const float (&A)[kRows][4], const float (&B)[kRows][4],
                                           Map (&e)[kRows]) {
  using Op = AffOp<false, Careful>;
  Map rw = identity_map();  // composition of the wave's earlier rows
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    Map c{A[r][0], B[r][0], 0u};
#pragma unroll
    for (int j = 1; j < 4; ++j) c = Op::compose(c, Map{A[r][j], B[r][j], 0u});
    wave_scan<Op>(c);
    if (!Careful) c.a = fix_underflow(c.a);
    e[r] = Op::compose(rw, prev_lane_map(c));  // everything before the lane's first item
    if (!Careful) e[r].a = fix_underflow(e[r].a);
    rw = COp::compose(rw, lane_map(c, 63));
  }
  return rw;
}

// Each element's composition from the tile start: q (everything before the
// lane's first item) followed by the lane's items in order.
template <bool Careful>
__device__ __forceinline__ void chain(const Map &q, const float (&A)[4], const float (&B)[4],
                                      bool nudge_zeros, float (&oa)[4], float (&ob)[4]) {
  using Op = AffOp<false, Careful>;
  Map m = q;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m = Op::compose(m, Map{A[j], B[j], 0u});
    if (!Careful && nudge_zeros) m.a = fix_underflow(m.a);
    oa[j] = m.a;
    ob[j] = m.b;
  }
}

// Whether the wave's multipliers include +-inf (same in every lane).
__device__ __forceinline__ uint32_t wave_has_inf(const float (&A)[kRows][4]) {
  bool inf = false;
#pragma unroll
  for (int r = 0; r < kRows; ++r)
#pragma unroll
    for (int j = 0; j < 4; ++j) inf = inf || __builtin_isinf(A[r][j]);
  return __builtin_amdgcn_ballot_w64(inf) != 0 ? 1u : 0u;
}

// seq[tile] = 1 marks a tile holding a multiplier of +-inf: the state after
// it depends on the sign of the state before it, which no affine map
// expresses, so the carry pass evaluates that tile element by element from
// its exact incoming value and the apply pass leaves it alone.
__global__ __launch_bounds__(kThreads) void local_kernel(const float *__restrict__ a,
                                                         const float *__restrict__ b,
                                                         float *__restrict__ pa,
                                                         float *__restrict__ pb,
                                                         float *__restrict__ agg,
                                                         uint32_t *__restrict__ seq, int64_t n) {
  __shared__ Map s_w[kWaves];
  __shared__ uint32_t s_inf[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  float A[kRows][4], B[kRows][4];
  const bool fast = load_rows(a, b, n, wave_start, A, B);
  Map e[kRows];
  const Map rw = fast ? rows_prefix<false>(A, B, e) : rows_prefix<true>(A, B, e);
  const uint32_t inf = fast ? 0u : wave_has_inf(A);  // a ballot: every lane takes part
  if (lane == 0) {
    s_w[wave] = rw;
    s_inf[wave] = inf;
  }
  __syncthreads();
  Map wa = identity_map();  // composition of the tile's earlier waves
  for (int w = 0; w < wave; ++w) wa = COp::compose(wa, s_w[w]);
  if (wave == kWaves - 1 && lane == 0) {
    const Map t = COp::compose(wa, rw);
    agg[2 * tile] = t.a;
    agg[2 * tile + 1] = t.b;
    uint32_t any = 0u;
    for (int w = 0; w < kWaves; ++w) any |= s_inf[w];
    seq[tile] = any;
  }
  // With earlier waves exactly zero (a zero multiplier there) every output
  // multiplier is exactly zero too; otherwise zeros are underflows.
  const bool nudge_zeros = wa.a != 0.0f;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const Map q = COp::compose(wa, e[r]);
    float oa[4], ob[4];
    if (fast)
      chain<false>(q, A[r], B[r], nudge_zeros, oa, ob);
    else
      chain<true>(q, A[r], B[r], false, oa, ob);
    store_rows(pa, pb, n, wave_start, r, oa, ob);
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

template <bool Careful>
__device__ __forceinline__ void hs_row(float (&A)[4], float (&B)[4], int lane) {
  using Op = AffOp<false, Careful>;
  auto comp = [](float xa, float xb, float ya, float yb, float &ra, float &rb) {
    const Map m = Op::compose(Map{xa, xb, 0u}, Map{ya, yb, 0u});
    ra = m.a;
    rb = m.b;
  };
  float nA[4], nB[4];
  {  // d = 1: element 4l+j reads 4l+j-1; item 0 reads the previous lane's item 3
    const float pa = shfl_up_f(A[3], 1), pb = shfl_up_f(B[3], 1);
    if (lane >= 1) comp(pa, pb, A[0], B[0], nA[0], nB[0]); else { nA[0] = A[0]; nB[0] = B[0]; }
#pragma unroll
    for (int j = 1; j < 4; ++j) comp(A[j - 1], B[j - 1], A[j], B[j], nA[j], nB[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) { A[j] = nA[j]; B[j] = nB[j]; }
  }
  {  // d = 2: items 0, 1 read the previous lane's items 2, 3
    const float pa2 = shfl_up_f(A[2], 1), pb2 = shfl_up_f(B[2], 1);
    const float pa3 = shfl_up_f(A[3], 1), pb3 = shfl_up_f(B[3], 1);
    if (lane >= 1) {
      comp(pa2, pb2, A[0], B[0], nA[0], nB[0]);
      comp(pa3, pb3, A[1], B[1], nA[1], nB[1]);
    } else {
      nA[0] = A[0]; nB[0] = B[0]; nA[1] = A[1]; nB[1] = B[1];
    }
    comp(A[0], B[0], A[2], B[2], nA[2], nB[2]);
    comp(A[1], B[1], A[3], B[3], nA[3], nB[3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) { A[j] = nA[j]; B[j] = nB[j]; }
  }
#pragma unroll
  for (int s = 1; s < 64; s *= 2) {  // d = 4s: the same item s lanes back
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float pa = shfl_up_f(A[j], s), pb = shfl_up_f(B[j], s);
      if (lane >= s) comp(pa, pb, A[j], B[j], nA[j], nB[j]); else { nA[j] = A[j]; nB[j] = B[j]; }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { A[j] = nA[j]; B[j] = nB[j]; }
  }
  if (!Careful) {
#pragma unroll
    for (int j = 0; j < 4; ++j) A[j] = fix_underflow(A[j]);
  }
}

// The wave's rows scanned in place (inclusive within each row); e[r] is the
// composition of the wave's rows before row r, the result the wave's total.
template <bool Careful>
__device__ __forceinline__ Map hs_rows(float (&A)[kRows][4], float (&B)[kRows][4],
                                       Map (&e)[kRows], int lane) {
  Map rw = identity_map();
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    hs_row<Careful>(A[r], B[r], lane);
    e[r] = rw;
    rw = COp::compose(rw, Map{lane_f(A[r][3], 63), lane_f(B[r][3], 63), 0u});
  }
  return rw;
}

__global__ __launch_bounds__(kThreads) void local_hs_kernel(const float *__restrict__ a,
                                                            const float *__restrict__ b,
                                                            float *__restrict__ pa,
                                                            float *__restrict__ pb,
                                                            float *__restrict__ agg,
                                                            uint32_t *__restrict__ seq, int64_t n) {
  __shared__ Map s_w[kWaves];
  __shared__ uint32_t s_inf[kWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t tile = blockIdx.x;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  float A[kRows][4], B[kRows][4];
  const bool fast = load_rows(a, b, n, wave_start, A, B);
  Map e[kRows];  // composition of the wave's rows before row r
  const uint32_t inf = fast ? 0u : wave_has_inf(A);  // before the rows are scanned in place
  const Map rw = fast ? hs_rows<false>(A, B, e, lane) : hs_rows<true>(A, B, e, lane);
  if (lane == 0) {
    s_w[wave] = rw;
    s_inf[wave] = inf;
  }
  __syncthreads();
  Map wa = identity_map();  // composition of the tile's earlier waves
  for (int w = 0; w < wave; ++w) wa = COp::compose(wa, s_w[w]);
  if (wave == kWaves - 1 && lane == 0) {
    const Map t = COp::compose(wa, rw);
    agg[2 * tile] = t.a;
    agg[2 * tile + 1] = t.b;
    uint32_t any = 0u;
    for (int w = 0; w < kWaves; ++w) any |= s_inf[w];
    seq[tile] = any;
  }
  // Fast waves: the row prefixes are finite and nudged (non-zero), so a zero
  // output multiplier is an underflow unless the earlier waves' multiplier
  // is exactly zero (then every output multiplier is).
  const bool nudge_zeros = wa.a != 0.0f;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const Map q = COp::compose(wa, e[r]);  // everything before the row
    float oa[4], ob[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Map o;
      if (fast) {
        o = FOp::compose(q, Map{A[r][j], B[r][j], 0u});
        if (nudge_zeros) o.a = fix_underflow(o.a);
      } else {
        o = COp::compose(q, Map{A[r][j], B[r][j], 0u});
      }
      oa[j] = o.a;
      ob[j] = o.b;
    }
    store_rows(pa, pb, n, wave_start, r, oa, ob);
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
// result is deterministic. Tile aggregates are mostly underflowed products,
// so every composition here is careful.
constexpr int kCarryThreads = 1024;
constexpr int kCarryWaves = kCarryThreads / 64;
constexpr int kBatch = 16;

// Rare path (a tile holds a multiplier of +-inf): one lane walks the tiles in
// order, pushing h through each ordinary tile's aggregate and through each
// marked tile element by element, writing that tile's outputs itself.
__device__ void carry_in_sequence(const float *__restrict__ agg,
                                  const uint32_t *__restrict__ seq, const float *__restrict__ a,
                                  const float *__restrict__ b, float *__restrict__ h,
                                  float *__restrict__ hin, float h0, int64_t ntiles, int64_t n) {
  float v = h0;
  for (int64_t t = 0; t < ntiles; ++t) {
    if (seq[t]) {
      const int64_t end = (t + 1) * kTileElems < n ? (t + 1) * kTileElems : n;
      for (int64_t i = t * kTileElems; i < end; ++i) {
        v = __builtin_fmaf(a[i], v, b[i]);
        h[i] = v;
      }
    } else {
      hin[t] = v;
      v = COp::apply(Map{agg[2 * t], agg[2 * t + 1], 0u}, v);
    }
  }
}

__global__ __launch_bounds__(kCarryThreads) void carry_kernel(const float *__restrict__ agg,
                                                              const uint32_t *__restrict__ seq,
                                                              const float *__restrict__ a,
                                                              const float *__restrict__ b,
                                                              float *__restrict__ out,
                                                              float *__restrict__ hin,
                                                              float h0, int64_t ntiles,
                                                              int64_t rows, int64_t n) {
  __shared__ Map s_w[kCarryWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Any tile marked? Four flags per 16-byte load (whole groups of four below
  // ntiles; the 0-3 left one by one), the loads of a thread in flight
  // together: with a short-circuit test per flag each load was a round trip
  // (the kernel took 18 against 9 us).
  uint32_t marked = 0u;
  const int64_t nvec = ntiles / 4;
  const uint4 *sv = reinterpret_cast<const uint4 *>(seq);
#pragma unroll 4
  for (int64_t v = threadIdx.x; v < nvec; v += kCarryThreads) {
    const uint4 f = sv[v];
    marked |= f.x | f.y | f.z | f.w;
  }
  for (int64_t t = nvec * 4 + threadIdx.x; t < ntiles; t += kCarryThreads) marked |= seq[t];
  if (__syncthreads_or(marked != 0u)) {
    if (threadIdx.x == 0) carry_in_sequence(agg, seq, a, b, out, hin, h0, ntiles, n);
    return;
  }
  const int64_t first = int64_t(wave) * rows;  // the wave's first row
  Map im[kBatch];                              // inclusive scans of a batch of rows
  // Rows k0 .. k0 + kBatch - 1 of the wave, each scanned across lanes; tiles
  // past the wave's rows or past the end are the identity.
  auto scan_batch = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int64_t t = (first + k0 + j) * 64 + lane;
      const int64_t tc = t < ntiles ? t : ntiles - 1;
      im[j] = Map{agg[2 * tc], agg[2 * tc + 1], 0u};
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const bool in = k0 + j < rows && (first + k0 + j) * 64 + lane < ntiles;
      if (!in) im[j] = identity_map();
      wave_scan<COp>(im[j]);
    }
  };
  Map tw = identity_map();  // the wave's total, the same in every lane
  for (int64_t k0 = 0; k0 < rows; k0 += kBatch) {
    scan_batch(k0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) tw = COp::compose(tw, lane_map(im[j], 63));
  }
  if (lane == 0) s_w[wave] = tw;
  __syncthreads();
  Map wa = identity_map();  // earlier waves
  for (int w = 0; w < wave; ++w) wa = COp::compose(wa, s_w[w]);
  float h = COp::apply(wa, h0);       // entering the wave's first row
  const bool cached = rows <= kBatch;  // same for every wave
  for (int64_t k0 = 0; k0 < rows; k0 += kBatch) {
    if (!cached) scan_batch(k0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const Map x = prev_lane_map(im[j]);  // earlier lanes of the row
      const int64_t t = (first + k0 + j) * 64 + lane;
      if (k0 + j < rows && t < ntiles) hin[t] = COp::apply(x, h);
      h = COp::apply(lane_map(im[j], 63), h);
    }
  }
}

// 1024 elements per workgroup (one float4 per thread); the tile's incoming
// value is wave-uniform.
__global__ __launch_bounds__(256) void apply_kernel(const float *__restrict__ pa,
                                                    const float *__restrict__ pb,
                                                    const float *__restrict__ hin,
                                                    const uint32_t *__restrict__ seq,
                                                    float *__restrict__ h, int64_t n) {
  const int64_t off = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t tile = (int64_t(blockIdx.x) * 1024) / kTileElems;
  if (seq[tile]) return;  // written by the carry pass
  const float c = hin[tile];
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
  return up(size_t(n) * 4) * 2 + up(size_t(ntiles) * 8) + up(size_t(ntiles) * 4) * 2;
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
  uint32_t *seq = reinterpret_cast<uint32_t *>(w + 2 * up(size_t(n) * 4) + up(size_t(ntiles) * 8) +
                                               up(size_t(ntiles) * 4));
  if (hillis_steele)
    hipLaunchKernelGGL(local_hs_kernel, dim3(unsigned(ntiles)), dim3(kThreads), 0, stream, a, b,
                       pa, pb, agg, seq, n);
  else
    hipLaunchKernelGGL(local_kernel, dim3(unsigned(ntiles)), dim3(kThreads), 0, stream, a, b, pa,
                       pb, agg, seq, n);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t rows = (ntiles + kCarryThreads - 1) / kCarryThreads;  // per wave, of 64 tiles
  hipLaunchKernelGGL(carry_kernel, dim3(1), dim3(kCarryThreads), 0, stream, agg, seq, a, b, h, hin,
                     h0, ntiles, rows, n);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int64_t groups = (n + 1023) / 1024;
  hipLaunchKernelGGL(apply_kernel, dim3(unsigned(groups)), dim3(256), 0, stream, pa, pb, hin, seq,
                     h, n);
  return hipGetLastError();
}

}  // namespace ssm
