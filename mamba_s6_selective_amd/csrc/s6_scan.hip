// S6 selective scan (forward, reverse, bidirectional) for gfx950.
//
// Computes, per (b, t, d, n) (POPCORNBENCH transcript FW-GLM-5-1, level 2
// problem 30, problem-statement forward pass):
//   dA = exp(delta*A), dBu = delta*u*B, h = dA*h + dBu (h starts at 0),
//   y[b,t,d] = sum_n C[b,t,n]*h[b,d,n] + D[d]*u[b,t,d],
// with the reverse recurrence running t downwards and the bidirectional form
// summing both ("ARM-Scan — Optimized Mamba Selective-Scan Kernel", "Approach").
//
// Layout: one lane per channel d (256 channels per workgroup); B[b,t,:] and
// C[b,t,:] are the same for every channel, so they are wave-uniform and reach
// the VALU through scalar loads and SGPR operands (no LDS, no VALU cost);
// u, delta and y move as coalesced per-lane words along d. The N-long state
// lives in VGPRs; dA, dBu and h never touch memory. exp(x) is evaluated as
// v_exp_f32(x * log2(e)) with log2(e) folded into A once per channel.
//
// The sequence is split into chunks so that enough lanes run (L-splitting):
//  1. chunk pass: every chunk runs its recurrence from a zero state, writes
//     its local y (with the D*u term), the sum of delta over the chunk per d
//     (the chunk's multiplier for state n is exp(A[d,n] * that sum)), the
//     local end state per (d, n) (reverse: the local state at the chunk
//     start) and small per-block statistics for the fix pass.
//  2. carry pass: per (b, n, d), a left fold over the chunk aggregates gives
//     each chunk's incoming state (forward and/or reverse); the fold is split
//     over waves (parts of 8 or 16 chunks) joined through LDS.
//  3. fix pass: every chunk except the first (forward) / last (reverse) adds
//     sum_n C[t,n] * carry_n * exp(A_n * S_t), S_t the running sum of delta
//     from the carry's entry point, to its y. This is the exact carry
//     contribution (the state is linear in its initial value). A group of
//     states whose terms are provably below 2^-24 for a whole block of steps
//     is left out (a truncated tail of a decaying series: at most 2^-22 per
//     output and direction, far inside the fp32 tolerance); blocks with no
//     group left are not touched at all.
// All three passes are deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "../../include/ssmscan.h"
#include "internal.h"
#include "s6_internal.h"

namespace ssm {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float ldv(const float *p) { return *p; }
__device__ __forceinline__ float ldv(const uint16_t *p) {
  return __uint_as_float(uint32_t(*p) << 16);
}
// A u or delta word as loaded (fp32 bits, or a bf16 value zero-extended),
// for words fetched a block of steps ahead: they are widened to fp32 only
// where they are used (widen). Widening at the load makes the wave wait for
// the load right there, which is what fetching ahead is meant to avoid.
__device__ __forceinline__ uint32_t ldw(const float *p) { return __float_as_uint(*p); }
__device__ __forceinline__ uint32_t ldw(const uint16_t *p) { return *p; }
template <typename T>
__device__ __forceinline__ float widen(uint32_t w) {
  return __uint_as_float(sizeof(T) == 2 ? w << 16 : w);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x with zero kept for x = -inf only. v_exp_f32 flushes results below 2^-126
// to zero; a state of +-inf multiplied by that zero would give NaN where the
// exact (tiny, non-zero) factor keeps it infinite, as the float64 recurrence
// does. Such a result becomes the smallest subnormal instead (for a finite
// state that changes the product by at most 2^-149 times the state).
__device__ __forceinline__ float exp2_nz(float x) {
  const float e = exp2_hw(x);
  return (e == 0.0f && x > -__builtin_inff()) ? __uint_as_float(1u) : e;
}
// x*y for factors that are non-negative or NaN (products of exponentials):
// a zero from two non-zero factors (an underflow) becomes the smallest
// subnormal, so "exactly zero" keeps meaning "a factor was exactly zero".
__device__ __forceinline__ float mul_pos_nz(float x, float y) {
  const float p = x * y;
  return (p == 0.0f && x != 0.0f && y != 0.0f) ? __uint_as_float(1u) : p;
}

// Waits for every outstanding scalar (and LDS) load. Scalar loads may return
// out of order, so a wait for one row is a wait for all; issuing it before the
// next step's row loads (rather than letting the compiler place it after them)
// keeps those loads in flight across the step.
__device__ __forceinline__ void wait_scalar_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0 (GFX9 encoding)
}

// Element at a wave-uniform base plus a per-lane 32-bit byte offset: lets the
// compiler use the scalar-base + 32-bit-offset form of global loads/stores
// instead of per-lane 64-bit address arithmetic on the VALU.
template <typename T>
__device__ __forceinline__ T &at(T *base, uint32_t byte_off) {
  return *reinterpret_cast<T *>(reinterpret_cast<char *>(base) + byte_off);
}
template <typename T>
__device__ __forceinline__ const T &at(const T *base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

// A B or C row (N values at a wave-uniform address) as raw words, so it can
// be loaded one step ahead into SGPRs and widened to fp32 only when used. bf16
// rows of even length are read as 32-bit words (two values each); the loads
// stay scalar and the widening (a shift or a mask) runs on the scalar unit.
template <typename T, int NT>
struct Row {
  static constexpr bool kPacked = sizeof(T) == 2 && NT % 2 == 0;
  static constexpr int kWords = kPacked ? NT / 2 : NT;
  uint32_t w[kWords];

  __device__ __forceinline__ void load(const T *__restrict__ p) {
    if constexpr (sizeof(T) == 4 || kPacked) {
      const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = q[i];
    } else {
#pragma unroll
      for (int i = 0; i < kWords; ++i) w[i] = uint32_t(p[i]) << 16;
    }
  }
  __device__ __forceinline__ float get(int n) const {
    if constexpr (kPacked)
      return __uint_as_float((n & 1) ? (w[n >> 1] & 0xffff0000u) : (w[n >> 1] << 16));
    else
      return __uint_as_float(w[n]);
  }
};

template <typename T, int NT>
__device__ __forceinline__ void load_row(const T *__restrict__ p, float (&out)[NT]) {
  Row<T, NT> r;
  r.load(p);
#pragma unroll
  for (int n = 0; n < NT; ++n) out[n] = r.get(n);
}

struct Geometry {
  int batch, L, d_inner, groups, nchunks, chunk;
  int nblk;      // blocks of kPrefetch steps in a full chunk
  int full_fix;  // 1: the fix pass evaluates every carry term (no skipped groups or blocks)
};

__device__ __forceinline__ void decompose(const Geometry &g, int &b, int &c, int &d) {
  const int bid = blockIdx.x;
  const int grp = bid % g.groups;
  const int rest = bid / g.groups;
  c = rest % g.nchunks;
  b = rest / g.nchunks;
  d = grp * kThreads + threadIdx.x;
}

// End-state / carry arrays are laid out [b][chunk][n][d] and delta sums
// [b][chunk][d], so lanes (d) are contiguous.
__device__ __forceinline__ size_t agg_index(const Geometry &g, int NT, int b, int c, int n,
                                            int d) {
  return ((size_t(b) * g.nchunks + c) * NT + n) * g.d_inner + d;
}
// Per-block statistics are laid out [b][chunk][block][d], block in the
// sweep order of their direction.
__device__ __forceinline__ size_t stat_index(const Geometry &g, int b, int c, int k, int d) {
  return ((size_t(b) * g.nchunks + c) * g.nblk + k) * g.d_inner + d;
}
__device__ __forceinline__ size_t sum_index(const Geometry &g, int b, int c, int d) {
  return (size_t(b) * g.nchunks + c) * g.d_inner + d;
}

constexpr int kPrefetch = 8;  // steps of u/delta (and y) kept in flight per lane
constexpr float kLn2 = 0.6931471805599453f;

// log(1 + e^x) = max(x, 0) + log(1 + e^-|x|): v_log_f32 on 1 + e^-|x|, or,
// where e^-|x| < 2^-6 and 1 + e^-|x| would round much of it away, the series
// e - e^2/2 + e^3/3 - e^4/4 (truncation below 2^-30 relative).
__device__ __forceinline__ float softplus_f(float x) {
  const float e = exp2_hw(-fabsf(x) * kLog2e);
  const float l = e < 0.015625f
                      ? e * (1.0f - e * (0.5f - e * (0.33333334f - 0.25f * e)))
                      : __builtin_amdgcn_logf(1.0f + e) * kLn2;
  return fmaxf(x, 0.0f) + l;
}

// What the scan does with each delta it reads: use it as given, or replace it
// by softplus(delta + bias[d]) (the transcript's delta = softplus(projection +
// bias), fused so that the activated delta never goes through memory).
struct DeltaAsIs {
  __device__ __forceinline__ float operator()(float x) const { return x; }
};
struct DeltaSoftplus {
  float bias;
  __device__ __forceinline__ float operator()(float x) const { return softplus_f(x + bias); }
};
template <class DX>
__device__ __forceinline__ DX make_dx(const float *bias, int d) {
  if constexpr (std::is_same<DX, DeltaSoftplus>::value)
    return DeltaSoftplus{bias ? bias[d] : 0.0f};
  else
    return DX{};
}

// One step of the chunk-local recurrence for one lane: returns y's value.
template <typename T, int NT, bool Careful = false>
__device__ __forceinline__ float s6_step(float dt, float x, const Row<T, NT> &Br,
                                         const Row<T, NT> &Cr, const float (&Ap)[NT],
                                         float Dd, float (&h)[NT]) {
  const float du = dt * x;
  // Two partial sums halve the dependent chain of output FMAs.
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float dA = Careful ? exp2_nz(dt * Ap[n]) : exp2_hw(dt * Ap[n]);
    h[n] = __builtin_fmaf(dA, h[n], du * Br.get(n));
    if (n & 1)
      acc1 = __builtin_fmaf(Cr.get(n), h[n], acc1);
    else
      acc0 = __builtin_fmaf(Cr.get(n), h[n], acc0);
  }
  return __builtin_fmaf(Dd, x, acc0 + acc1);
}

// What one direction's chunk sweep leaves for the fix pass, per full block of
// kPrefetch steps (sweep order): the running delta sum at the block's end
// and the block's smallest running sum (a NaN sum stays NaN), both exact.
// Reads one element per 64 bytes of the B and C rows of one block of steps
// (first_elem: element offset of the block's lowest row), lanes 0-31 in B and
// 32-63 in C, so that those lines are on their way to L2 before the scalar
// loads of the block ask for them. The value means nothing; holding it until
// a later point (keep_alive) is what keeps the loads.
template <typename T, int NT>
__device__ __forceinline__ uint32_t touch_rows(const T *__restrict__ B, const T *__restrict__ C,
                                               size_t first_elem) {
  constexpr int kElems = kPrefetch * NT;
  constexpr int kStride = 64 / int(sizeof(T));
  const int lane = int(__lane_id());
  const T *base = lane < 32 ? B : C;
  const int i = min((lane & 31) * kStride, kElems - 1);
  const T v = base[first_elem + size_t(i)];
  if constexpr (sizeof(T) == 4)
    return __float_as_uint(v);
  else
    return uint32_t(v);
}
__device__ __forceinline__ void keep_alive(uint32_t v) { asm volatile("" ::"v"(v)); }
// Marks x as rewritten here (no instruction), so that the computation of x
// stays before this point instead of moving to its uses.
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

struct SweepStats {
  float *s_end;
  float *s_min;
};

// One sweep of the chunk-local recurrence from a zero state. Writes (or, when
// Accumulate, adds) y for every step of the chunk, the block statistics in
// st (when st.s_min is set), and leaves the final state in h and the sum of
// delta in S. Steps run in blocks of kPrefetch with no
// branch inside a block (so the compiler can overlap neighbouring steps), and
// each lane's words for the next block are loaded while the current block
// computes; B[t] and C[t] are wave-uniform scalar loads. A tail of fewer than
// kPrefetch steps runs one step at a time, with exp2_nz.
// Returns true (the same in every lane) when a block's exponential may have
// flushed to zero: then y, h and S are not to be used, and careful_sweep
// evaluates the chunk again (the statistics stand: they depend on delta alone).
template <typename T, int NT, bool Reverse, bool Accumulate, class DX>
__device__ __forceinline__ bool chunk_sweep(const T *__restrict__ u, const T *__restrict__ delta,
                                            const T *__restrict__ B, const T *__restrict__ C,
                                            float *__restrict__ y, const float (&Ap)[NT],
                                            float Dd, const DX &dx, const Geometry &g, int b,
                                            int c, int d, int t0, int t1, float (&h)[NT],
                                            float &S, const SweepStats &st) {
#pragma unroll
  for (int n = 0; n < NT; ++n) h[n] = 0.0f;
  S = 0.0f;
  float ap_min = Ap[0];  // the most negative exponent factor of the lane
#pragma unroll
  for (int n = 1; n < NT; ++n) ap_min = fminf(ap_min, Ap[n]);
  const size_t row0 = size_t(b) * g.L;
  const int len = t1 - t0;
  const int full = len - len % kPrefetch;
  auto tof = [&](int i) { return Reverse ? (t1 - 1 - i) : (t0 + i); };
  auto row = [&](int i) { return (row0 + tof(i)) * size_t(g.d_inner); };
  const uint32_t io = uint32_t(d) * uint32_t(sizeof(T));  // input byte offset of the lane
  const uint32_t yo = uint32_t(d) * 4u;                    // output byte offset of the lane
  // The lane's statistics addresses, formed once: they hold the channel, so
  // they sit in VGPRs and leave the scalar registers to the B/C rows.
  const size_t ss = size_t(g.d_inner);
  const bool stats = st.s_min != nullptr;
  float *pe = stats ? st.s_end + stat_index(g, b, c, 0, d) : nullptr;
  float *pw = stats ? st.s_min + stat_index(g, b, c, 0, d) : nullptr;
  // Two register sets for a block's delta, u (and y) words: one feeds the
  // block being computed while the next block's loads land in the other,
  // and the loop runs two blocks per iteration so the sets trade roles
  // without copies.
  // The delta and u words stay as loaded until the block that uses them
  // widens them (ldw, widen).
  uint32_t ad[kPrefetch], ax[kPrefetch], bd[kPrefetch], bx[kPrefetch];
  float ay[kPrefetch], by[kPrefetch];
  // Lowest row of the block of steps starting at sweep index i.
  auto block_row = [&](int i) { return row0 + tof(Reverse ? i + kPrefetch - 1 : i); };
  uint32_t touched = 0;
  bool flushes = false;  // this lane's deltas may flush an exponential to zero
  if (full > 0) {
    touched = touch_rows<T, NT>(B, C, block_row(0) * NT);
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const size_t r = row(j);
      ad[j] = ldw(&at(delta + r, io));
      ax[j] = ldw(&at(u + r, io));
      if (Accumulate) ay[j] = at(y + r, yo);
    }
  }
  // One block of kPrefetch steps from sweep index i0, its words in (rd, rx,
  // cy); the next block's words are loaded into (nd, nx, ny).
  auto block = [&](int i0, const uint32_t (&rd)[kPrefetch], const uint32_t (&rx)[kPrefetch],
                   const float (&cy)[kPrefetch], uint32_t (&nd)[kPrefetch],
                   uint32_t (&nx)[kPrefetch], float (&ny)[kPrefetch]) {
    // Widened and transformed when used: their loads have had a block of
    // steps to land. The u words are widened here (pinned), not next to a
    // use that comes after the next block's loads.
    float cd[kPrefetch], cx[kPrefetch];
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      cd[j] = dx(widen<T>(rd[j]));
      cx[j] = widen<T>(rx[j]);
      pin(cx[j]);
    }
    // A step's exponential can flush to zero only if delta*A*log2(e) < -126
    // (|delta*A| > 87); noted per block from the largest delta (an infinite
    // one included), before the next block's loads are issued, so the wait
    // for this block's words is not a wait for those. Such a chunk is
    // evaluated again step by step (careful_sweep): a branch to a step-by-step
    // block here cost the common path registers.
    float dmax = cd[0];
#pragma unroll
    for (int j = 1; j < kPrefetch; ++j) dmax = fmaxf(dmax, cd[j]);
    flushes = flushes || dmax * ap_min < -126.0f;
    keep_alive(touched);  // issued a block ago, with the words just consumed
    if (i0 + kPrefetch < full) {
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j) {
        const size_t rn = row(i0 + kPrefetch + j);
        nd[j] = ldw(&at(delta + rn, io));
        nx[j] = ldw(&at(u + rn, io));
        if (Accumulate) ny[j] = at(y + rn, yo);
      }
      touched = touch_rows<T, NT>(B, C, block_row(i0 + kPrefetch) * NT);
    }
    float smin = 0.0f;
    // B/C rows go one step ahead: step j's rows were loaded during step j-1.
    Row<T, NT> Bc, Cc;
    Bc.load(B + (row0 + tof(i0)) * NT);
    Cc.load(C + (row0 + tof(i0)) * NT);
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      Row<T, NT> Bn, Cn;
      wait_scalar_loads();
      if (j + 1 < kPrefetch) {
        Bn.load(B + (row0 + tof(i0 + j + 1)) * NT);
        Cn.load(C + (row0 + tof(i0 + j + 1)) * NT);
      }
      // Keeps the next rows' loads at the head of the step: left to itself the
      // scheduler may sink them (with their address arithmetic) to just before
      // the next wait, which then waits for the whole scalar-load latency.
      __builtin_amdgcn_sched_barrier(0);
      const float out = s6_step<T, NT>(cd[j], cx[j], Bc, Cc, Ap, Dd, h);
      at(y + row(i0 + j), yo) = Accumulate ? cy[j] + out : out;
      S += cd[j];
      smin = j == 0 ? S : fminf(smin, S);
      if (j + 1 < kPrefetch) {
        Bc = Bn;
        Cc = Cn;
      }
    }
    if (stats) {  // wave-uniform
      // A NaN in the running sum reaches the block's end; fminf would drop it.
      *pe = S;
      *pw = S == S ? smin : S;
      pe += ss;
      pw += ss;
    }
  };
  for (int i0 = 0; i0 < full; i0 += 2 * kPrefetch) {
    block(i0, ad, ax, ay, bd, bx, by);
    if (i0 + kPrefetch >= full) break;
    block(i0 + kPrefetch, bd, bx, by, ad, ax, ay);
  }
  for (int i = full; i < len; ++i) {
    const size_t r = row(i);
    const float dt = dx(ldv(&at(delta + r, io)));
    const float x = ldv(&at(u + r, io));
    const int t = tof(i);
    Row<T, NT> Bc, Cc;
    Bc.load(B + (row0 + t) * NT);
    Cc.load(C + (row0 + t) * NT);
    const float out = s6_step<T, NT, true>(dt, x, Bc, Cc, Ap, Dd, h);
    float &yr = at(y + r, yo);
    yr = Accumulate ? yr + out : out;
    S += dt;
  }
  return __builtin_amdgcn_ballot_w64(flushes) != 0;
}

// The chunk-local recurrence from a zero state, step by step with exp2_nz,
// so that an infinite state stays infinite as in the float64 recurrence
// where a fast sweep's exponential may have flushed to zero (rare: delta*|A|
// above 87 in the chunk). The same arithmetic as chunk_sweep otherwise, so
// the same y, h and S.
template <typename T, int NT, bool Reverse, bool Accumulate, class DX>
__device__ __forceinline__ void careful_sweep(const T *__restrict__ u,
                                              const T *__restrict__ delta,
                                              const T *__restrict__ B, const T *__restrict__ C,
                                              float *__restrict__ y, const float (&Ap)[NT],
                                              float Dd, const DX &dx, const Geometry &g, int b,
                                              int d, int t0, int t1, float (&h)[NT], float &S) {
#pragma unroll
  for (int n = 0; n < NT; ++n) h[n] = 0.0f;
  S = 0.0f;
  const size_t row0 = size_t(b) * g.L;
  const uint32_t io = uint32_t(d) * uint32_t(sizeof(T));
  const uint32_t yo = uint32_t(d) * 4u;
#pragma unroll 1
  for (int i = 0; i < t1 - t0; ++i) {
    const int t = Reverse ? (t1 - 1 - i) : (t0 + i);
    const size_t r = (row0 + t) * size_t(g.d_inner);
    const float dt = dx(ldv(&at(delta + r, io)));
    Row<T, NT> Bc, Cc;
    Bc.load(B + (row0 + t) * NT);
    Cc.load(C + (row0 + t) * NT);
    const float out = s6_step<T, NT, true>(dt, ldv(&at(u + r, io)), Bc, Cc, Ap, Dd, h);
    float &yr = at(y + r, yo);
    yr = Accumulate ? yr + out : out;
    S += dt;
  }
}

template <typename T, int NT, class DX>
__global__ __launch_bounds__(kThreads, 4) void s6_chunk_kernel(
    const T *__restrict__ u, const T *__restrict__ delta, const float *__restrict__ dbias,
    const float *__restrict__ A,
    const T *__restrict__ B, const T *__restrict__ C, const float *__restrict__ D,
    float *__restrict__ y, float *__restrict__ agg_s, float *__restrict__ agg_f,
    float *__restrict__ agg_r, float *__restrict__ sf_end, float *__restrict__ sf_min,
    float *__restrict__ sr_end, float *__restrict__ sr_min, Geometry g, int direction) {
  int b, c, d;
  decompose(g, b, c, d);
  if (d >= g.d_inner) return;
  const int t0 = c * g.chunk;
  const int t1 = min(g.L, t0 + g.chunk);
  float Ap[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) Ap[n] = A[size_t(d) * NT + n] * kLog2e;
  const float Dd = D[d];
  const DX dx = make_dx<DX>(dbias, d);
  float h[NT];
  float S = 0.0f;
  const bool multi = g.nchunks > 1;
  // Statistics for the fix pass, which runs only with several chunks.
  const SweepStats stf{sf_end, multi ? sf_min : nullptr};
  const SweepStats str{sr_end, multi ? sr_min : nullptr};
  if (direction != SSM_DIR_REV) {
    if (chunk_sweep<T, NT, false, false>(u, delta, B, C, y, Ap, Dd, dx, g, b, c, d, t0, t1, h,
                                         S, stf))
      careful_sweep<T, NT, false, false>(u, delta, B, C, y, Ap, Dd, dx, g, b, d, t0, t1, h, S);
    if (multi) {
      agg_s[sum_index(g, b, c, d)] = S;
#pragma unroll
      for (int n = 0; n < NT; ++n) agg_f[agg_index(g, NT, b, c, n, d)] = h[n];
    }
  }
  if (direction != SSM_DIR_FWD) {
    if (direction == SSM_DIR_BIDIR) {
      if (chunk_sweep<T, NT, true, true>(u, delta, B, C, y, Ap, Dd, dx, g, b, c, d, t0, t1, h,
                                         S, str)) {
        // The sweep has added to y what it must not have: y is formed again
        // by the forward sweep, then the reverse one adds its own.
        float hf[NT], sf;
        careful_sweep<T, NT, false, false>(u, delta, B, C, y, Ap, Dd, dx, g, b, d, t0, t1, hf,
                                           sf);
        careful_sweep<T, NT, true, true>(u, delta, B, C, y, Ap, Dd, dx, g, b, d, t0, t1, h, S);
      }
    } else if (chunk_sweep<T, NT, true, false>(u, delta, B, C, y, Ap, Dd, dx, g, b, c, d, t0, t1,
                                               h, S, str)) {
      careful_sweep<T, NT, true, false>(u, delta, B, C, y, Ap, Dd, dx, g, b, d, t0, t1, h, S);
    }
    if (multi) {
      if (direction == SSM_DIR_REV) agg_s[sum_index(g, b, c, d)] = S;
#pragma unroll
      for (int n = 0; n < NT; ++n) agg_r[agg_index(g, NT, b, c, n, d)] = h[n];
    }
  }
}

// Per (b, n, d): incoming state of every chunk, by a left fold of the chunk
// aggregates (forward: chunk 0 upwards; reverse: last chunk down). A block
// covers 64 channels (lanes) of one (b, n); wave p owns chunks
// [p*Part, (p+1)*Part) in both directions, holds their multipliers and end
// states in registers, and folds them into part totals; the totals meet in
// LDS, and each wave then replays its chunks from the fold of the totals
// before it (forward: lower parts; reverse: higher parts). Part is 8 chunks
// when that covers the sequence with at most kCarryMaxParts waves, else
// kCarryPart: short sequences get more, shorter waves (measured faster on
// 32-chunk sequences). Fixed shapes, so the result is deterministic.
constexpr int kCarryPart = 16;      // the largest part
constexpr int kCarryMaxParts = 16;  // so at most 256 chunks

template <int Part>
__global__ __launch_bounds__(64 * kCarryMaxParts) void s6_carry_kernel(
    const float *__restrict__ agg_s, const float *__restrict__ agg_f,
    const float *__restrict__ agg_r, const float *__restrict__ A, float *__restrict__ carry_f,
    float *__restrict__ carry_r, Geometry g, int NT, int direction) {
  __shared__ float s_a[kCarryMaxParts][64], s_f[kCarryMaxParts][64], s_r[kCarryMaxParts][64];
  const int lane = threadIdx.x & 63;
  const int part = threadIdx.x >> 6;
  const int parts = blockDim.x >> 6;
  const int dgroups = (g.d_inner + 63) / 64;
  int bid = blockIdx.x;
  const int dg = bid % dgroups;
  bid /= dgroups;
  const int n = bid % NT;
  const int b = bid / NT;
  const int d = dg * 64 + lane;
  const bool valid = d < g.d_inner;
  const bool fwd = direction != SSM_DIR_REV, rev = direction != SSM_DIR_FWD;
  const int k0 = part * Part;
  // All loads first, from indices clamped into range (lanes past d_inner and
  // chunks past the end read valid entries whose values are then replaced),
  // so that they are in flight together: a load under a per-lane condition
  // whose value feeds an exp in the same branch would be waited for one at a
  // time.
  const int dc = valid ? d : 0;
  const float Aval = A[size_t(dc) * NT + n];
  float ra[Part], rf[Part] = {}, rr[Part] = {};
#pragma unroll
  for (int i = 0; i < Part; ++i)
    ra[i] = agg_s[sum_index(g, b, min(k0 + i, g.nchunks - 1), dc)];
  if (fwd) {
#pragma unroll
    for (int i = 0; i < Part; ++i)
      rf[i] = agg_f[agg_index(g, NT, b, min(k0 + i, g.nchunks - 1), n, dc)];
  }
  if (rev) {
#pragma unroll
    for (int i = 0; i < Part; ++i)
      rr[i] = agg_r[agg_index(g, NT, b, min(k0 + i, g.nchunks - 1), n, dc)];
  }
  const float Ap = valid ? Aval * kLog2e : 0.0f;
#pragma unroll
  for (int i = 0; i < Part; ++i) {
    const bool in = valid && k0 + i < g.nchunks;  // chunks past the end act as identity maps
    ra[i] = in ? exp2_nz(Ap * ra[i]) : 1.0f;
    rf[i] = in && fwd ? rf[i] : 0.0f;
    rr[i] = in && rev ? rr[i] : 0.0f;
  }
  float ta = 1.0f, tf = 0.0f, tr = 0.0f;
#pragma unroll
  for (int i = 0; i < Part; ++i) {
    tf = __builtin_fmaf(ra[i], tf, rf[i]);
    tr = __builtin_fmaf(ra[Part - 1 - i], tr, rr[Part - 1 - i]);
    ta = mul_pos_nz(ta, ra[i]);
  }
  s_a[part][lane] = ta;
  s_f[part][lane] = tf;
  s_r[part][lane] = tr;
  __syncthreads();
  float cf = 0.0f, cr = 0.0f;
  for (int q = 0; q < part; ++q) cf = __builtin_fmaf(s_a[q][lane], cf, s_f[q][lane]);
  for (int q = parts - 1; q > part; --q) cr = __builtin_fmaf(s_a[q][lane], cr, s_r[q][lane]);
#pragma unroll
  for (int i = 0; i < Part; ++i) {
    const int k = k0 + i;
    if (fwd && valid && k < g.nchunks) carry_f[agg_index(g, NT, b, k, n, d)] = cf;
    cf = __builtin_fmaf(ra[i], cf, rf[i]);
  }
#pragma unroll
  for (int i = Part - 1; i >= 0; --i) {
    const int k = k0 + i;
    if (rev && valid && k < g.nchunks) carry_r[agg_index(g, NT, b, k, n, d)] = cr;
    cr = __builtin_fmaf(ra[i], cr, rr[i]);
  }
}

// Carry contribution at one step: sum_n C[t,n] * cin[n] * exp(A[n] * S).
// The carry's terms decay: with A[d,n] < 0 and the running delta sum S
// growing, cin[n] * exp(A[d,n] * S) shrinks, and the tail of this decaying
// sum is truncated with a proven bound.
//
// States go in groups of kFixGroup. For a group g, Ag = its largest Ap[n]
// (the slowest decay; Ap = A * log2(e)) and Smin >= 0 the smallest running
// sum over a block of kPrefetch steps, every term of the group at every step
// of the block is at most maxC * sum_{n in g} |cin[n]| * 2^(Ag * Smin)
// (2^(Ap[n] * S_j) <= 2^(Ag * S_j) <= 2^(Ag * Smin) for Ap[n] <= Ag < 0 and
// S_j >= Smin), maxC the largest |C| over the chunk. When that bound, times a
// margin for its own rounding and the hardware exp2's error, is at most
// kTruncGroup in every lane, the group is left out of the block: with at
// most 4 groups (N <= 16) the output changes by at most 2^-22 per direction
// (fp32's own rounding of a unit-sized y is 2^-24). Carries that are not
// finite, NaN exponent factors and non-negative ones are never left out, nor
// is anything of a block whose running sum can be negative or NaN (there the
// bound does not hold); a term whose exponential is exactly zero falls under
// the rule like any other.
constexpr int kFixGroup = 4;
constexpr float kTruncGroup = 0x1p-24f;
constexpr float kTruncScale = 1.01f / kTruncGroup;  // margin / kTruncGroup

template <int NT>
struct FixGroups {
  static constexpr int kCount = (NT + kFixGroup - 1) / kFixGroup;
  float Ag[kCount];     // largest Ap[n] of the group
  float cabs[kCount];   // sum of |cin[n]| over the group
  bool keep[kCount];    // never left out: a non-finite carry, a NaN or non-negative Ap
  float sdead[kCount];  // smallest running sum at which the group was left out (NaN: never)
  __device__ __forceinline__ FixGroups(const float (&Ap)[NT], const float (&cin)[NT]) {
#pragma unroll
    for (int g = 0; g < kCount; ++g) {
      sdead[g] = __builtin_nanf("");
      float ag = -__builtin_inff(), ca = 0.0f;
      bool k = false;
#pragma unroll
      for (int i = 0; i < kFixGroup; ++i) {
        const int n = g * kFixGroup + i;
        if (n < NT) {
          ag = fmaxf(ag, Ap[n]);
          ca += fabsf(cin[n]);
          k = k || !__builtin_isfinite(cin[n]) || Ap[n] != Ap[n];
        }
      }
      Ag[g] = ag;
      cabs[g] = ca;
      keep[g] = k || !(ag < 0.0f);
    }
  }
  // Decides a block of kPrefetch steps from the chunk pass's smallest
  // running sum over it: bit g set when group g has a lane that needs its
  // terms (0: the block leaves y as it is). cscale = maxC * kTruncScale.
  // Blocks are decided in sweep order. The bound only shrinks as the
  // smallest running sum grows (cabs, Ag < 0 and cscale are fixed for the
  // sweep), so a group left out at smallest sum s stays out for a block
  // whose smallest sum is at least s in every lane, without its
  // exponential; otherwise (a negative delta, a NaN) the bound is evaluated.
  __device__ __forceinline__ uint32_t decide(float smin, float cscale) {
    const bool ok = smin >= 0.0f;  // false for a NaN or a negative sum
    uint32_t m = 0;
#pragma unroll
    for (int g = 0; g < kCount; ++g) {
      if (__builtin_amdgcn_ballot_w64(!(smin >= sdead[g])) == 0) continue;  // still out
      const float bound = cabs[g] * exp2_hw(Ag[g] * smin) * cscale;
      const bool drop = ok && !keep[g] && bound <= 1.0f;  // false for a NaN bound
      if (__builtin_amdgcn_ballot_w64(!drop) != 0)
        m |= 1u << g;
      else
        sdead[g] = fminf(sdead[g], smin);  // fminf(NaN, s) = s
    }
    return m;
  }
};

// Largest mag(p[i]) over i in [0, count), each lane of the wave's active
// lanes (a prefix of the wave) taking every nact-th item; four loads per lane
// are in flight at a time (one at a time would cost a memory round trip per
// item a lane reads).
template <class V, class Mag>
__device__ __forceinline__ uint32_t lanes_max(const V *__restrict__ p, size_t count, Mag mag) {
  const size_t lane = __lane_id();
  const size_t nact = size_t(__popcll(__builtin_amdgcn_read_exec()));
  uint32_t m = 0;
  for (size_t i0 = lane; i0 < count; i0 += 4 * nact) {
    V r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const size_t i = i0 + k * nact;
      r[k] = i < count ? p[i] : V{};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, mag(r[k]));
  }
  return m;
}

// The largest |C| over the chunk's C rows [first, first + count) (element
// offsets, whole rows) as an fp32 bit pattern (0x7f800000 or more: a NaN or
// an infinity), the same in every lane: the magnitudes, as bit patterns,
// reduced over the wave's active lanes and then wave-wide with an unsigned
// max. Rows of whole 16-byte vectors (C is 16-byte aligned) are read as
// vectors, bf16 rows of even length as pairs.
template <typename T, int NT>
__device__ __forceinline__ uint32_t chunk_cmax_bits(const T *__restrict__ C, size_t first,
                                                    size_t count) {
  auto mag32 = [](uint32_t x) -> uint32_t {  // a 32-bit word: one fp32 or two bf16
    if constexpr (sizeof(T) == 2)
      return max((x << 16) & 0x7fffffffu, x & 0x7fff0000u);
    else
      return x & 0x7fffffffu;
  };
  uint32_t m;
  if constexpr (NT * sizeof(T) % 16 == 0) {
    m = lanes_max(reinterpret_cast<const uint4 *>(C + first), count * sizeof(T) / 16,
                  [&](const uint4 &v) {
                    return max(max(mag32(v.x), mag32(v.y)), max(mag32(v.z), mag32(v.w)));
                  });
  } else if constexpr (sizeof(T) == 2 && NT % 2 == 0) {
    m = lanes_max(reinterpret_cast<const uint32_t *>(C + first), count / 2, mag32);
  } else if constexpr (sizeof(T) == 2) {
    m = lanes_max(C + first, count,
                  [](uint16_t x) { return (uint32_t(x) << 16) & 0x7fffffffu; });
  } else {
    m = lanes_max(reinterpret_cast<const uint32_t *>(C + first), count, mag32);
  }
  return __ockl_wfred_max_u32(m);
}
// maxC * kTruncScale from those bits (+inf for a non-finite C).
__device__ __forceinline__ float cscale_of(uint32_t m) {
  return m >= 0x7f800000u ? __builtin_inff() : __uint_as_float(m) * kTruncScale;
}

template <typename T, int NT, bool Gated, bool Careful>
__device__ __forceinline__ float fix_step(float S, const Row<T, NT> &Cr, const float (&Ap)[NT],
                                          const float (&cin)[NT], uint32_t live) {
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int g = 0; g < FixGroups<NT>::kCount; ++g) {
    if (Gated && !((live >> g) & 1u)) continue;  // wave-uniform
#pragma unroll
    for (int i = 0; i < kFixGroup; ++i) {
      const int n = g * kFixGroup + i;
      if (n < NT) {
        const float v = cin[n] * (Careful ? exp2_nz(Ap[n] * S) : exp2_hw(Ap[n] * S));
        if (n & 1)
          acc1 = __builtin_fmaf(Cr.get(n), v, acc1);
        else
          acc0 = __builtin_fmaf(Cr.get(n), v, acc0);
      }
    }
  }
  return acc0 + acc1;
}

// Blocks whose statistics words are decided together; the words of the next
// window are loaded while the current one is worked on.
constexpr int kFixWindow = 8;

// The fix pass over one chunk in one direction. Blocks are decided from the
// chunk pass's statistics, a window at a time, without touching delta or y;
// delta, y and the running sum before the block are loaded only for blocks
// that change y, the next such block's while the current one computes. The
// running sums start from the chunk pass's exact values, so every step sees
// the same sum the sequential sweep would. A tail of fewer than kPrefetch
// steps is always evaluated in full. cscale is cscale_of the chunk's largest
// |C| (finite here).
template <typename T, int NT, bool Reverse, class DX>
__device__ __forceinline__ void fix_sweep(const T *__restrict__ delta, const T *__restrict__ C,
                                          float *__restrict__ y, const float (&Ap)[NT],
                                          const float (&cin)[NT], const DX &dx,
                                          const Geometry &g, int b, int c, int d, int t0,
                                          int t1, float cscale, const float *__restrict__ s_end,
                                          const float *__restrict__ s_min) {
  const size_t row0 = size_t(b) * g.L;
  const int len = t1 - t0;
  const int nfull = len / kPrefetch;
  const int full = nfull * kPrefetch;
  auto tof = [&](int i) { return Reverse ? (t1 - 1 - i) : (t0 + i); };
  auto row = [&](int i) { return (row0 + tof(i)) * size_t(g.d_inner); };
  const uint32_t io = uint32_t(d) * uint32_t(sizeof(T));
  const uint32_t yo = uint32_t(d) * 4u;
  const size_t s0 = stat_index(g, b, c, 0, d);
  const size_t ss = size_t(g.d_inner);  // stride between blocks of the statistics
  FixGroups<NT> groups(Ap, cin);
  // A non-finite carry (rare): every step with every group, one step at a
  // time with exp2_nz, so that an infinite carry times an exponential that
  // flushed to zero stays infinite; the running sum is formed again from the
  // chunk's entry point (the same additions as the chunk pass, so the same
  // sums). Kept out of the loop below, where a branch to it cost registers.
  bool nonfinite = false;
#pragma unroll
  for (int n = 0; n < NT; ++n) nonfinite = nonfinite || !__builtin_isfinite(cin[n]);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(nonfinite) != 0, 0)) {
    float S = 0.0f;
#pragma unroll 1
    for (int i = 0; i < len; ++i) {
      const size_t r = row(i);
      S += dx(ldv(&at(delta + r, io)));
      Row<T, NT> Cc;
      Cc.load(C + (row0 + tof(i)) * NT);
      float &yr = at(y + r, yo);
      yr = yr + fix_step<T, NT, false, true>(S, Cc, Ap, cin, 0);
    }
    return;
  }
  // The words one live block needs: its delta words (widened when the block
  // runs), its y words, the running sum before it, and the value of a load
  // that brings its C rows toward L2 ahead of its scalar row loads (held
  // until the block runs).
  struct Words {
    uint32_t d[kPrefetch];
    float yv[kPrefetch];
    float s_in;
    uint32_t touched;
  };
  auto load_block = [&](int k, Words &w) {
    w.touched = touch_rows<T, NT>(
        C, C, (row0 + tof(Reverse ? k * kPrefetch + kPrefetch - 1 : k * kPrefetch)) * NT);
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      w.d[j] = ldw(&at(delta + row(k * kPrefetch + j), io));
      w.yv[j] = at(y + row(k * kPrefetch + j), yo);
    }
    w.s_in = k > 0 ? s_end[s0 + size_t(k - 1) * ss] : 0.0f;
  };
  // Takes up a block's words (the running sum at each of its steps, its y
  // words): the waits for its loads fall here.
  auto take_up = [&](Words &w, float (&Sj)[kPrefetch], float (&yv)[kPrefetch]) {
    float S = w.s_in;  // the running sum before the block
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      S += dx(widen<T>(w.d[j]));
      Sj[j] = S;
      pin(Sj[j]);
      yv[j] = w.yv[j];
      pin(yv[j]);
    }
    keep_alive(w.touched);
  };
  // Evaluates block k from its taken-up values for the groups in live.
  auto run_block = [&](int k, const float (&Sj)[kPrefetch], const float (&yv)[kPrefetch],
                       uint32_t live) {
    const int i0 = k * kPrefetch;
    Row<T, NT> Cc;
    Cc.load(C + (row0 + tof(i0)) * NT);
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      Row<T, NT> Cn;
      wait_scalar_loads();
      if (j + 1 < kPrefetch) Cn.load(C + (row0 + tof(i0 + j + 1)) * NT);
      at(y + row(i0 + j), yo) = yv[j] + fix_step<T, NT, true, false>(Sj[j], Cc, Ap, cin, live);
      if (j + 1 < kPrefetch) Cc = Cn;
    }
  };

  float wn[kFixWindow];  // smallest running sums of the next window's blocks
#pragma unroll
  for (int i = 0; i < kFixWindow; ++i) wn[i] = i < nfull ? s_min[s0 + size_t(i) * ss] : 0.0f;
  for (int w0 = 0; w0 < nfull; w0 += kFixWindow) {
    // Decide the window: 4 bits of live groups per block.
    uint32_t masks = 0;
#pragma unroll
    for (int i = 0; i < kFixWindow; ++i) {
      if (w0 + i < nfull) {
        const uint32_t m = g.full_fix ? 0xfu : groups.decide(wn[i], cscale);
        masks |= m << (4 * i);
      }
    }
#pragma unroll
    for (int i = 0; i < kFixWindow; ++i) {
      const int k = w0 + kFixWindow + i;
      if (k < nfull) wn[i] = s_min[s0 + size_t(k) * ss];
    }
    if (masks == 0) continue;  // wave-uniform: the whole window leaves y as it is
    // Its blocks that change y, each one's words loaded while the one before
    // it computes and taken up after that one's stores, the one way into
    // that point, so that its waits count those stores and wait for its own
    // loads alone.
    int i = __builtin_ctz(masks) / 4;
    Words w;
    float Sj[kPrefetch], yv[kPrefetch];
    load_block(w0 + i, w);
    take_up(w, Sj, yv);
    for (;;) {
      const uint32_t live = (masks >> (4 * i)) & 0xfu;
      masks &= ~(0xfu << (4 * i));
      const int inext = masks ? __builtin_ctz(masks) / 4 : -1;
      if (inext >= 0) load_block(w0 + inext, w);
      run_block(w0 + i, Sj, yv, live);
      if (inext < 0) break;
      i = inext;
      take_up(w, Sj, yv);
    }
  }
  float S = nfull > 0 ? s_end[s0 + size_t(nfull - 1) * ss] : 0.0f;
  for (int i = full; i < len; ++i) {
    const size_t r = row(i);
    S += dx(ldv(&at(delta + r, io)));
    Row<T, NT> Cc;
    Cc.load(C + (row0 + tof(i)) * NT);
    float &yr = at(y + r, yo);
    yr = yr + fix_step<T, NT, false, true>(S, Cc, Ap, cin, 0);
  }
}

// A chunk whose C rows hold an inf or NaN: y = sum_n C*(local state + carry
// term) cannot be had as the chunk pass's sum_n C*(local state) plus a
// correction sum_n C*(carry term) when C is infinite (inf*x + inf*z where the
// recurrence forms inf*(x + z)). Such a chunk is evaluated again from its
// exact incoming states, step by step, in each direction the call computes
// (y overwritten: the forward sweep writes its output with D*u, the reverse
// sweep adds its own), with exp2_nz. Only inputs with a non-finite C take
// this path.
template <typename T, int NT, class DX>
__device__ void recompute_chunk(const T *__restrict__ u, const T *__restrict__ delta,
                                const T *__restrict__ B, const T *__restrict__ C,
                                const float (&Ap)[NT], float Dd, const DX &dx,
                                const float *__restrict__ carry_f,
                                const float *__restrict__ carry_r, float *__restrict__ y,
                                const Geometry &g, int b, int c, int d, int t0, int t1,
                                int direction) {
  const size_t row0 = size_t(b) * g.L;
  const uint32_t io = uint32_t(d) * uint32_t(sizeof(T));
  const uint32_t yo = uint32_t(d) * 4u;
  auto run = [&](auto reverse, const float *carry, bool has_carry, bool accumulate) {
    constexpr bool kRev = decltype(reverse)::value;
    float h[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) h[n] = has_carry ? carry[agg_index(g, NT, b, c, n, d)] : 0.0f;
#pragma unroll 1
    for (int i = 0; i < t1 - t0; ++i) {
      const int t = kRev ? t1 - 1 - i : t0 + i;
      const size_t r = (row0 + t) * size_t(g.d_inner);
      Row<T, NT> Bc, Cc;
      Bc.load(B + (row0 + t) * NT);
      Cc.load(C + (row0 + t) * NT);
      const float out = s6_step<T, NT, true>(dx(ldv(&at(delta + r, io))), ldv(&at(u + r, io)),
                                             Bc, Cc, Ap, Dd, h);
      float &yr = at(y + r, yo);
      yr = accumulate ? yr + out : out;
    }
  };
  if (direction != SSM_DIR_REV)
    run(std::false_type{}, carry_f, c > 0, false);
  if (direction != SSM_DIR_FWD)
    run(std::true_type{}, carry_r, c < g.nchunks - 1, direction == SSM_DIR_BIDIR);
}

template <typename T, int NT, class DX>
__global__ __launch_bounds__(kThreads, 4) void s6_fix_kernel(
    const T *__restrict__ u, const T *__restrict__ delta, const float *__restrict__ dbias,
    const float *__restrict__ A, const T *__restrict__ B, const T *__restrict__ C,
    const float *__restrict__ D, float *__restrict__ y, const float *__restrict__ carry_f,
    const float *__restrict__ carry_r, const float *__restrict__ sf_end,
    const float *__restrict__ sf_min, const float *__restrict__ sr_end,
    const float *__restrict__ sr_min, Geometry g, int direction) {
  int b, c, d;
  decompose(g, b, c, d);
  if (d >= g.d_inner) return;
  const bool do_f = direction != SSM_DIR_REV && c > 0;
  const bool do_r = direction != SSM_DIR_FWD && c < g.nchunks - 1;
  if (!do_f && !do_r) return;
  const int t0 = c * g.chunk;
  const int t1 = min(g.L, t0 + g.chunk);
  float Ap[NT], cin[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) Ap[n] = A[size_t(d) * NT + n] * kLog2e;
  const DX dx = make_dx<DX>(dbias, d);
  const uint32_t cmax =
      chunk_cmax_bits<T, NT>(C, (size_t(b) * g.L + t0) * NT, size_t(t1 - t0) * NT);
  if (__builtin_expect(cmax >= 0x7f800000u, 0)) {  // wave-uniform: C holds an inf or NaN
    recompute_chunk<T, NT, DX>(u, delta, B, C, Ap, D[d], dx, carry_f, carry_r, y, g, b, c, d,
                               t0, t1, direction);
    return;
  }
  const float cscale = cscale_of(cmax);
  if (do_f) {
#pragma unroll
    for (int n = 0; n < NT; ++n) cin[n] = carry_f[agg_index(g, NT, b, c, n, d)];
    fix_sweep<T, NT, false>(delta, C, y, Ap, cin, dx, g, b, c, d, t0, t1, cscale, sf_end,
                            sf_min);
  }
  if (do_r) {
#pragma unroll
    for (int n = 0; n < NT; ++n) cin[n] = carry_r[agg_index(g, NT, b, c, n, d)];
    fix_sweep<T, NT, true>(delta, C, y, Ap, cin, dx, g, b, c, d, t0, t1, cscale, sr_end,
                           sr_min);
  }
}

// Chunk length (a multiple of 8): the largest power-of-two number of chunks
// per sequence whose (batch, chunk, channel-group) workgroups the GPU holds
// at once (one round, so every workgroup starts together and none waits for
// a second round), chunks of at least 32 steps (shorter ones leave the carry
// no room to decay, so the fix pass redoes nearly all the work: 16-step
// chunks measured 10 % slower on a 1024-step sequence), at most
// kCarryPart * kCarryMaxParts chunks per sequence. Filling every resident
// slot instead measured 2-6 % slower on each of the four shapes tried where
// the two differ: every chunk boundary adds fix-pass work.
// SSMSCAN_S6_CHUNK overrides the length (still within the chunk-count limit).
int plan_chunk(int batch, int L, int groups, int resident_wgs) {
  const int64_t max_chunks = kCarryPart * kCarryMaxParts;
  int64_t chunk = 0;
  if (const char *env = getenv("SSMSCAN_S6_CHUNK")) chunk = atoi(env);
  if (chunk <= 0) {
    const int64_t rows = int64_t(batch) * groups;
    const int64_t fit = resident_wgs / rows;
    int64_t nch = 1;
    while (2 * nch <= fit) nch *= 2;
    chunk = (L + nch - 1) / nch;
    if (chunk < 32) chunk = 32;
  }
  if (chunk < (L + max_chunks - 1) / max_chunks) chunk = (L + max_chunks - 1) / max_chunks;
  chunk = (chunk + 7) / 8 * 8;
  return int(chunk);
}

// Workgroups of the chunk kernel resident on the whole device at once.
template <typename T, int NT, class DX>
int resident_chunk_wgs() {
  static int cached = 0;
  if (cached > 0) return cached;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, s6_chunk_kernel<T, NT, DX>, kThreads,
                                                   0) != hipSuccess ||
      cus <= 0 || per_cu <= 0)
    return 1024;
  cached = cus * per_cu;
  return cached;
}

template <typename T, int NT, class DX>
int launch_all(const S6Args &a, hipStream_t stream) {
  Geometry g;
  g.batch = a.batch;
  g.L = a.L;
  g.d_inner = a.d_inner;
  g.groups = (a.d_inner + kThreads - 1) / kThreads;
  g.chunk = plan_chunk(a.batch, a.L, g.groups, resident_chunk_wgs<T, NT, DX>());
  // SSMSCAN_S6_FULL_FIX=1 turns the fix pass's truncation off (every carry
  // term evaluated), to check the truncation's bound and to time the
  // untruncated cost.
  const char *full = getenv("SSMSCAN_S6_FULL_FIX");
  g.full_fix = (full && atoi(full) != 0) ? 1 : 0;
  g.nchunks = (a.L + g.chunk - 1) / g.chunk;
  g.nblk = g.chunk / kPrefetch;
  const int64_t wgs = int64_t(g.groups) * g.nchunks * a.batch;
  if (wgs > (int64_t(1) << 31) - 1) return fail(SSM_ERR_UNSUPPORTED, "problem too large");

  float *agg_s = nullptr, *agg_f = nullptr, *agg_r = nullptr, *car_f = nullptr,
        *car_r = nullptr, *sf_end = nullptr, *sr_end = nullptr, *sf_min = nullptr,
        *sr_min = nullptr;
  if (g.nchunks > 1) {
    const size_t per = size_t(a.batch) * g.nchunks * NT * a.d_inner;
    const size_t sums = (size_t(a.batch) * g.nchunks * a.d_inner + 63) / 64 * 64;
    const size_t stats = (size_t(a.batch) * g.nchunks * g.nblk * a.d_inner + 63) / 64 * 64;
    void *buf = nullptr;
    if (int rc = s6_workspace(stream, (4 * per + sums + 4 * stats) * sizeof(float), &buf))
      return rc;
    float *f = static_cast<float *>(buf);
    agg_s = f;
    agg_f = f + sums;
    agg_r = agg_f + per;
    car_f = agg_r + per;
    car_r = car_f + per;
    sf_end = car_r + per;
    sf_min = sf_end + stats;
    sr_end = sf_end + 2 * stats;
    sr_min = sf_end + 3 * stats;
  }
  const T *u = static_cast<const T *>(a.u);
  const T *dl = static_cast<const T *>(a.delta);
  const T *B = static_cast<const T *>(a.B);
  const T *C = static_cast<const T *>(a.C);
  hipLaunchKernelGGL((s6_chunk_kernel<T, NT, DX>), dim3(unsigned(wgs)), dim3(kThreads), 0, stream,
                     u, dl, a.delta_bias, a.A, B, C, a.D, a.y, agg_s, agg_f, agg_r, sf_end,
                     sf_min, sr_end, sr_min, g, a.direction);
  if (int rc = hip_check(hipGetLastError(), "s6 chunk launch")) return rc;
  if (g.nchunks == 1) return SSM_OK;
  const int64_t carry_blocks = int64_t(a.batch) * NT * ((a.d_inner + 63) / 64);
  auto carry = [&](auto kernel, int part) {
    const int parts = (g.nchunks + part - 1) / part;
    hipLaunchKernelGGL(kernel, dim3(unsigned(carry_blocks)), dim3(64 * parts), 0, stream, agg_s,
                       agg_f, agg_r, a.A, car_f, car_r, g, NT, a.direction);
  };
  if (g.nchunks <= 8 * kCarryMaxParts)
    carry(s6_carry_kernel<8>, 8);
  else
    carry(s6_carry_kernel<kCarryPart>, kCarryPart);
  if (int rc = hip_check(hipGetLastError(), "s6 carry launch")) return rc;
  hipLaunchKernelGGL((s6_fix_kernel<T, NT, DX>), dim3(unsigned(wgs)), dim3(kThreads), 0, stream,
                     u, dl, a.delta_bias, a.A, B, C, a.D, a.y, car_f, car_r, sf_end, sf_min,
                     sr_end, sr_min, g, a.direction);
  return hip_check(hipGetLastError(), "s6 fix launch");
}

template <typename T, class DX>
int dispatch_n(const S6Args &a, hipStream_t s) {
  switch (a.N) {
#define SSM_CASE(K) \
  case K:           \
    return launch_all<T, K, DX>(a, s);
    SSM_CASE(1) SSM_CASE(2) SSM_CASE(3) SSM_CASE(4) SSM_CASE(5) SSM_CASE(6) SSM_CASE(7)
    SSM_CASE(8) SSM_CASE(9) SSM_CASE(10) SSM_CASE(11) SSM_CASE(12) SSM_CASE(13)
    SSM_CASE(14) SSM_CASE(15) SSM_CASE(16)
#undef SSM_CASE
    default:
      return fail(SSM_ERR_UNSUPPORTED, "N must be in 1..16");
  }
}

}  // namespace

int run_s6(const S6Args &a, hipStream_t stream) {
  if (a.delta_softplus)
    return a.bf16 ? dispatch_n<uint16_t, DeltaSoftplus>(a, stream)
                  : dispatch_n<float, DeltaSoftplus>(a, stream);
  return a.bf16 ? dispatch_n<uint16_t, DeltaAsIs>(a, stream)
                : dispatch_n<float, DeltaAsIs>(a, stream);
}

}  // namespace ssm
