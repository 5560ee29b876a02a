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
//  * the kernel is persistent; workgroups claim tiles in increasing order from
//    a ticket counter, so a tile only ever waits for lower tiles that running
//    workgroups own, and the lowest unfinished tile can always finish (no
//    assumption about how many workgroups are resident). Each workgroup has
//    four data waves, which load the next tile while the current one waits,
//    and one control wave that claims, publishes and looks back.
//  * data moves with non-temporal 16-byte loads and stores (read once, written
//    once), which measured about 8% faster than default caching here.
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

// Streaming (non-temporal) 16-byte loads and stores: a, b and h are touched
// exactly once, so they should not displace anything in L2 or the MALL.
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float *p) {
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(float *p, float4 o) {
  const v4f v = {o.x, o.y, o.z, o.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(p));
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

// Composition of the superblocks of this block before the current one: the
// level-1 words of all but the last (n1_old of them), then the last one
// composed from its 64 level-0 words (lanes 0..62 by the window scan, lane 63
// on top) -- the same operations its own last tile performs to publish it.
__device__ __forceinline__ void superblock_prefix(uint64_t w1a, uint64_t w1b, int n1_old,
                                                  uint64_t wpa, uint64_t wpb, bool use_prev,
                                                  int lane, float &pa, float &pb) {
  window_total(payload(w1a), payload(w1b), n1_old, lane, pa, pb);
  if (use_prev) {
    float qa, qb;
    window_total(payload(wpa), payload(wpb), kFan - 1, lane, qa, qb);
    const float la = lane_f(payload(wpa), kFan - 1), lb = lane_f(payload(wpb), kFan - 1);
    const float ta = qa * la, tb = __builtin_fmaf(la, qb, lb);  // previous superblock
    pb = __builtin_fmaf(ta, pb, tb);
    pa = pa * ta;
  }
}

// Incoming value of `tile`, composed from published aggregates (see the file
// comment): P2 over the level-2 words of earlier blocks, P1 over the level-1
// words of earlier superblocks of this block, P0 over the level-0 words of
// earlier tiles of this superblock. The superblock just before this one is
// not read from level 1 (its word is published by its last tile's look-back,
// one round trip later than its tiles' own words) but composed here from its
// 64 level-0 words with exactly the arithmetic its last tile uses to publish
// it, so both give the same bits. The last tile of a superblock publishes the
// superblock's aggregate, and the last tile of a block the block's aggregate,
// as soon as their inputs are visible. Called by all 64 lanes of one wave.
__device__ float look_back(const LinearStatus &st, int64_t tile, float ga, float gb, float h0,
                           uint32_t epoch, int lane) {
  const int64_t sb = tile / kFan;             // superblock of this tile
  const int64_t blk = sb / kFan;              // block of this tile
  const int n0 = int(tile - sb * kFan);       // level-0 words before the tile in its superblock
  const int n1 = int(sb - blk * kFan);        // superblocks before this one in its block
  const int n2 = int(blk);                    // blocks before this one
  const bool use_prev = n1 > 0;               // previous superblock composed from level 0
  const int n1_old = use_prev ? n1 - 1 : 0;   // level-1 words read
  const bool last_in_sb = n0 == kFan - 1;
  const bool last_in_blk = last_in_sb && n1 == kFan - 1;
  const int64_t i0 = sb * kFan + lane, ip = (sb - 1) * kFan + lane;
  const int64_t i1 = blk * kFan + lane, i2 = lane;
  uint64_t w0a = 0, w0b = 0, wpa = 0, wpb = 0, w1a = 0, w1b = 0, w2a = 0, w2b = 0;
  bool r0 = !(lane < n0), rp = !use_prev, r1 = !(lane < n1_old), r2 = !(lane < n2);
  bool pub1 = !last_in_sb, pub2 = !last_in_blk;
  float sa = 1.0f, sbv = 0.0f;  // this superblock's aggregate, when published here
  for (;;) {
    if (!r0) {
      w0a = ld_status(&st.lvl0[i0].a);
      w0b = ld_status(&st.lvl0[i0].b);
      r0 = word_ready(w0a, epoch) && word_ready(w0b, epoch);
    }
    if (!rp) {
      wpa = ld_status(&st.lvl0[ip].a);
      wpb = ld_status(&st.lvl0[ip].b);
      rp = word_ready(wpa, epoch) && word_ready(wpb, epoch);
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
    const bool all0 = __ballot(!r0) == 0, allp = __ballot(!rp) == 0;
    const bool all1 = __ballot(!r1) == 0, all2 = __ballot(!r2) == 0;
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
    if (!pub2 && pub1 && all1 && allp) {
      float p1a, p1b;
      superblock_prefix(w1a, w1b, n1_old, wpa, wpb, use_prev, lane, p1a, p1b);
      if (lane == 0) {
        st_status(&st.lvl2[blk].a, epoch, p1a * sa);
        st_status(&st.lvl2[blk].b, epoch, __builtin_fmaf(sa, p1b, sbv));
      }
      pub2 = true;
    }
    if (all0 && allp && all1 && all2 && pub1 && pub2) break;
    __builtin_amdgcn_s_sleep(1);
  }
  float p0a, p0b, p1a, p1b, p2a, p2b;
  window_total(payload(w0a), payload(w0b), n0, lane, p0a, p0b);
  superblock_prefix(w1a, w1b, n1_old, wpa, wpb, use_prev, lane, p1a, p1b);
  window_total(payload(w2a), payload(w2b), n2, lane, p2a, p2b);
  const float h2 = __builtin_fmaf(p2a, h0, p2b);
  const float h1 = __builtin_fmaf(p1a, h2, p1b);
  return __builtin_fmaf(p0a, h1, p0b);
}

// Loads one tile (rows of float4 per wave); past n the identity map (1, 0).
__device__ __forceinline__ void load_tile(const float *__restrict__ a,
                                          const float *__restrict__ b, int64_t n, int64_t tile,
                                          float4 (&va)[kRows], float4 (&vb)[kRows]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  if ((tile + 1) * kTileElems <= n) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t off = wave_start + r * kRowElems + lane * 4;
      va[r] = load_nt(a + off);
      vb[r] = load_nt(b + off);
    }
  } else {
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
}

// Data waves, phase 1: chunk aggregates of the lane's 4 items per row, a wave
// scan per row, and the wave's aggregate (rows folded in order) into LDS.
__device__ __forceinline__ void tile_local_scan(const float4 (&va)[kRows],
                                                const float4 (&vb)[kRows], float (&ia)[kRows],
                                                float (&ib)[kRows], float *s_wave_a,
                                                float *s_wave_b) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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
}

// Data waves, phase 2: carry into each row, then into each lane's chunk, then
// re-run the recurrence over the lane's 4 items and store.
__device__ __forceinline__ void tile_apply(const float4 (&va)[kRows], const float4 (&vb)[kRows],
                                           const float (&ia)[kRows], const float (&ib)[kRows],
                                           float c, float *__restrict__ h, int64_t n,
                                           int64_t tile) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  const bool full = (tile + 1) * kTileElems <= n;
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
      store_nt(h + off, o);
    } else {
      const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (off + j < n) h[off + j] = ov[j];
    }
    c = lane_f(end, 63);
  }
}

constexpr int kClaimTiles = 1;  // consecutive tiles taken per ticket (see the kernel comment)

__device__ __forceinline__ int64_t claim_batch(unsigned long long *ticket, int lane) {
  unsigned long long t = 0;
  if (lane == 0)
    t = __hip_atomic_fetch_add(ticket, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(t));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(t >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// The tile a workgroup scans after tile t: the next tile of its claimed batch,
// or the first tile of a newly claimed batch. ntiles means "none".
__device__ __forceinline__ int64_t successor(int64_t t, int64_t ntiles,
                                             unsigned long long *ticket, int lane) {
  if (t >= ntiles) return ntiles;
  if ((t + 1) % kClaimTiles != 0) return t + 1 < ntiles ? t + 1 : ntiles;
  const int64_t first = claim_batch(ticket, lane) * kClaimTiles;
  return first < ntiles ? first : ntiles;
}

// LDS shared by the waves of one workgroup. Everything one iteration hands
// across a barrier is double-buffered by iteration parity: a wave may run one
// iteration ahead of another between two barriers, and must not overwrite a
// value the other still has to read.
struct Shared {
  float wave_a[2][kWaves], wave_b[2][kWaves];  // per-wave aggregates
  float tile_a[2], tile_b[2];                  // tile aggregates
  float carry[2][kWaves];                      // h entering each wave's rows
  int64_t first[2];                            // first two claimed tiles
  int64_t after[2];                            // tile claimed for the iteration after next
  unsigned arrived[2];                         // data waves done with a tile's local scan
};

// Data waves: local scan of a loaded tile; the last data wave to finish folds
// the wave aggregates into the tile aggregate and publishes it (level 0) at
// once, without waiting for any other workgroup.
__device__ __forceinline__ void scan_and_publish(const float4 (&va)[kRows],
                                                 const float4 (&vb)[kRows], float (&ia)[kRows],
                                                 float (&ib)[kRows], Shared &sh, int slot,
                                                 const LinearStatus &st, int64_t tile,
                                                 uint32_t epoch) {
  const int lane = threadIdx.x & 63;
  tile_local_scan(va, vb, ia, ib, sh.wave_a[slot], sh.wave_b[slot]);
  unsigned prior = 0;
  if (lane == 0)
    prior = __hip_atomic_fetch_add(&sh.arrived[slot], 1u, __ATOMIC_ACQ_REL,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
  prior = __builtin_amdgcn_readfirstlane(prior);
  if (prior == kWaves - 1) {
    float ga = sh.wave_a[slot][0], gb = sh.wave_b[slot][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      gb = __builtin_fmaf(sh.wave_a[slot][w], gb, sh.wave_b[slot][w]);
      ga *= sh.wave_a[slot][w];
    }
    if (lane == 0) {
      st_status(&st.lvl0[tile].a, epoch, ga);
      st_status(&st.lvl0[tile].b, epoch, gb);
      sh.tile_a[slot] = ga;
      sh.tile_b[slot] = gb;
      sh.arrived[slot] = 0;  // reused two tiles later, after two barriers
    }
  }
}

// Persistent kernel. Workgroups claim tiles from a ticket counter, so tiles
// are claimed in increasing order and every claimed tile belongs to a running
// workgroup that scans its tiles in increasing order. Tiles are claimed one
// per ticket: with batches of consecutive tiles, a batch's later tiles are
// published only after an earlier look-back of the same workgroup, which
// chains the batches' last tiles one after another (measured: 2 tiles per
// ticket 1.75x slower, 4 tiles per ticket fully serialised).
//
// Within a workgroup, four data waves and one control wave overlap two tiles:
// while the control wave runs the look-back of tile c_i (whose aggregate was
// published one iteration earlier), the data waves load tile c_{i+1}, claim
// c_{i+2}, scan c_{i+1} and publish its aggregate; then the data waves apply
// c_i's carries and store it. Publishing a tile therefore never waits for its own workgroup's
// previous look-back to finish, which would chain every tile's publication to
// the look-back of an earlier tile. The control wave issues no data loads, so
// its status reads never queue behind outstanding data loads (the vector
// memory counter retires in order).
//
// Every wait is for something a lower tile produces before it waits on
// anything itself (level-0 aggregates right after its local scan, higher
// levels from the look-back of a lower tile), and a workgroup only waits on
// tiles lower than the ones it owns; so the lowest unfinished tile can always
// finish, however many workgroups the device keeps resident.
// The ticket of a launch is st.ticket[epoch & 1]; the first workgroup zeroes
// the other slot for the next launch on the stream.
__global__ __launch_bounds__(kThreads + 64) void linear_scan_kernel(
    const float *__restrict__ a, const float *__restrict__ b, float h0,
    float *__restrict__ h, int64_t n, int64_t ntiles, LinearStatus st, uint32_t epoch) {
  __shared__ Shared sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned long long *ticket = st.ticket + (epoch & 1u);

  if (wave == kWaves) {
    if (blockIdx.x == 0 && lane == 0)
      __hip_atomic_store(st.ticket + ((epoch + 1u) & 1u), 0ull, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    int64_t cur = claim_batch(ticket, lane) * kClaimTiles;
    if (cur > ntiles) cur = ntiles;
    int64_t nxt = successor(cur, ntiles, ticket, lane);
    if (lane == 0) {
      sh.first[0] = cur;
      sh.first[1] = nxt;
      sh.arrived[0] = 0;
      sh.arrived[1] = 0;
    }
    __syncthreads();  // A: first claims visible
    __syncthreads();  // B: first tile scanned and published
    for (int slot = 0; cur < ntiles; slot ^= 1) {
      const float ga = sh.tile_a[slot], gb = sh.tile_b[slot];
      const float h_in = look_back(st, cur, ga, gb, h0, epoch, lane);
      if (lane == 0) {
        float c = h_in;
        for (int w = 0; w < kWaves; ++w) {
          sh.carry[slot][w] = c;
          c = __builtin_fmaf(sh.wave_a[slot][w], c, sh.wave_b[slot][w]);
        }
      }
      __syncthreads();  // C: carries of `cur`, tile after `nxt`, `nxt` published
      cur = nxt;
      nxt = sh.after[slot];
    }
    return;
  }

  __syncthreads();  // A
  int64_t cur = sh.first[0], nxt = sh.first[1];
  float4 va[kRows], vb[kRows];
  float ia[kRows], ib[kRows];
  if (cur < ntiles) {
    load_tile(a, b, n, cur, va, vb);
    scan_and_publish(va, vb, ia, ib, sh, 0, st, cur, epoch);
  }
  __syncthreads();  // B
  for (int slot = 0; cur < ntiles; slot ^= 1) {
    float4 na[kRows], nb[kRows];
    float nia[kRows], nib[kRows];
    if (nxt < ntiles) {
      load_tile(a, b, n, nxt, na, nb);
      // Wave 0 finds (claiming if needed) the tile after `nxt`; a claim's
      // latency overlaps the loads it was queued behind, not the look-back.
      if (wave == 0) {
        const int64_t after = successor(nxt, ntiles, ticket, lane);
        if (lane == 0) sh.after[slot] = after;
      }
      scan_and_publish(na, nb, nia, nib, sh, slot ^ 1, st, nxt, epoch);
    } else if (wave == 0 && lane == 0) {
      sh.after[slot] = ntiles;
    }
    __syncthreads();  // C
    tile_apply(va, vb, ia, ib, sh.carry[slot][wave], h, n, cur);
    const int64_t after = sh.after[slot];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      va[r] = na[r];
      vb[r] = nb[r];
      ia[r] = nia[r];
      ib[r] = nib[r];
    }
    cur = nxt;
    nxt = after;
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
  hipLaunchKernelGGL(linear_scan_kernel, dim3(grid), dim3(kThreads + 64), 0, stream, a, b, h0,
                     h, n, ntiles, status, epoch);
  return hipGetLastError();
}

int linear_wgs_per_cu() {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(linear_scan_kernel), kThreads + 64, 0) !=
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
