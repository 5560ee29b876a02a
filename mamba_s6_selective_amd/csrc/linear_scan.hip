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
// L2s, where a status read that must see other XCDs' writes takes several
// microseconds while HBM is streaming:
//
//  * tile = 8 data waves x 4 rows x 64 lanes x float4 = 8192 elements (the
//    batched form: 11 waves x 3 rows = 8448, see Shape). Each row
//    is read and written with one fully coalesced 1 KiB global_load/store_dwordx4
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
//    composition of level-2, level-1 and level-0 windows of at most 64 words
//    each, each window composed by one fixed-shape wave64 DPP scan; the most
//    recent superblocks are read at level 0, so a look-back never waits on
//    another look-back that runs at the same time.
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
//    its data waves and one control wave, and a tile moves through a
//    four-stage pipeline (load, scan and publish, look-back, apply and store)
//    in which every long-latency step -- a tile's loads, the status reads of
//    its look-back -- is issued one iteration before its result is used.
//  * data moves with non-temporal 16-byte loads and stores (read once, written
//    once), which measured about 8% faster than default caching here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "internal.h"
#include "scan_common.h"

namespace ssm {
namespace {

constexpr int kRowElems = 256;  // 64 lanes x float4
constexpr int kFan = 64;        // entries per look-back window

// Tile shape: data waves per workgroup and float4 rows per wave. One
// sequence: 8 x 4 rows = 8192 elements. The batched form spends more VALU per
// element (segment positions, heads) and is fastest with more, shorter waves,
// 11 x 3 rows = 8448 elements (as many waves as fit the register file, with
// the parked tiles within LDS; 8 x 4: 320 against 301 us at 2^27, 9 x 4:
// 312, 10 x 3: 306); for one sequence that shape is no faster.
template <bool Seg>
struct Shape {
  static constexpr int kWaves = Seg ? 11 : 8;
  static constexpr int kRows = Seg ? 3 : 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWaveElems = kRowElems * kRows;
  static constexpr int kTileElems = kWaveElems * kWaves;
};

using namespace scan;

// Status words: bits 63..32 hold the launch's epoch (bit 63 of the multiplier
// word: the aggregate holds a sequence head, batched scans only), bits 31..0
// the fp32 payload. Epochs stay below 2^31.
constexpr uint64_t kHeadBit = uint64_t(1) << 63;

__device__ __forceinline__ uint64_t ld_status(const uint64_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_status(uint64_t *p, uint32_t epoch, float v,
                                          uint32_t head = 0u) {
  const uint64_t w = (uint64_t(epoch) << 32) | uint64_t(__float_as_uint(v)) |
                     (head ? kHeadBit : uint64_t(0));
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_map(AggWord &w, uint32_t epoch, const Map &m) {
  st_status(&w.a, epoch, m.a, m.head);
  st_status(&w.b, epoch, m.b);
}
__device__ __forceinline__ Map word_map(uint64_t wa, uint64_t wb) {
  return Map{__uint_as_float(uint32_t(wa)), __uint_as_float(uint32_t(wb)),
             (wa & kHeadBit) ? 1u : 0u};
}

__device__ __forceinline__ bool word_ready(uint64_t w, uint32_t epoch) {
  return (uint32_t(w >> 32) & 0x7fffffffu) == epoch;
}

// Composition, in lane order, of the maps held by lanes [0, count) of the
// wave (later lanes contribute the identity), returned in every lane. A fixed
// shape: the result depends only on the values and `count`.
//  window_total: plain products in one DPP tree;
//  window_total_careful: Op's rule (mul_nz products, heads honoured). With
//    all values finite that is the plain tree, with the head bits or-ed and a
//    multiplier that underflowed to zero nudged (unless a lane holds an exact
//    zero; a head's multiplier is exactly zero, so plain products already
//    drop what precedes it). Otherwise a loop of cross-lane shuffles, one
//    copy of the code (unrolled DPP steps at every window doubled the control
//    wave's code and slowed the scan through instruction fetch).
__device__ __forceinline__ Map window_total(Map m, int count, int lane) {
  if (lane >= count) m = identity_map();
  wave_scan<AffOp<false, false>>(m);
  return lane_map(m, 63);
}
template <class Op>
__device__ __forceinline__ Map window_total_careful(Map m, int count, int lane) {
  if (lane >= count) m = identity_map();
  const bool odd = !__builtin_isfinite(m.a) || !__builtin_isfinite(m.b);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(odd) == 0, 1)) {
    const bool zero = __builtin_amdgcn_ballot_w64(m.a == 0.0f) != 0;
    const uint32_t head = __builtin_amdgcn_ballot_w64(m.head != 0u) != 0 ? 1u : 0u;
    wave_scan<AffOp<false, false>>(m);
    Map t = lane_map(m, 63);
    if (t.a == 0.0f && !zero) t.a = nudge(t.a);
    t.head = head;
    return t;
  }
#pragma unroll 1
  for (int d = 1; d < 64; d *= 2) {
    Map p;
    p.a = __shfl_up(m.a, d);
    p.b = __shfl_up(m.b, d);
    p.head = uint32_t(__shfl_up(int(m.head), d));
    if (lane >= d) m = Op::compose(p, m);
  }
  return lane_map(m, 63);
}

// Look-back windows at level 0: the tile's own superblock and the
// kRecent - 1 superblocks before it. Older superblocks are read at level 1 and
// older blocks at level 2, but the words of those recent superblocks (and of
// the block they may straddle into) come from look-backs that may still be
// running when this one starts, so they are composed here from level-0 words.
constexpr int kRecent = 6;

// Resumable look-back of one tile: which words it reads, the words read so
// far and, per lane, whether that lane's word is complete. The tile's prefix
// is  (level-2 words of blocks [0, blk1)) (+) (level-1 words of superblocks
// [blk1*64, sb0)) (+) (level-0 windows of superblocks sb0 .. sb, the last one
// cut at the tile).
struct LookBack {
  int64_t sb0, blk1;
  int nw, n0, n1, n2;
  uint64_t wa[kRecent], wb[kRecent], w1a, w1b, w2a, w2b;
  bool r[kRecent], r1, r2;
};

__device__ __forceinline__ void lb_init(LookBack &s, int64_t tile, int lane) {
  const int64_t sb = tile / kFan;
  s.n0 = int(tile - sb * kFan);
  s.sb0 = sb >= kRecent - 1 ? sb - (kRecent - 1) : 0;
  s.nw = int(sb - s.sb0) + 1;
  s.blk1 = s.sb0 / kFan;
  s.n1 = int(s.sb0 - s.blk1 * kFan);
  s.n2 = int(s.blk1);
#pragma unroll
  for (int q = 0; q < kRecent; ++q) {
    const int entries = q < s.nw - 1 ? kFan : (q == s.nw - 1 ? s.n0 : 0);
    s.r[q] = !(lane < entries);
    s.wa[q] = 0;
    s.wb[q] = 0;
  }
  s.r1 = !(lane < s.n1);
  s.r2 = !(lane < s.n2);
  s.w1a = s.w1b = s.w2a = s.w2b = 0;
}

// One round of status reads for the words not yet complete. The loads are
// only issued here; lb_check reads them, so the reads of two look-backs can
// be in flight together.
__device__ __forceinline__ void lb_issue(LookBack &s, const LinearStatus &st, int lane) {
#pragma unroll
  for (int q = 0; q < kRecent; ++q) {
    if (!s.r[q]) {
      const int64_t i = (s.sb0 + q) * kFan + lane;
      s.wa[q] = ld_status(&st.lvl0[i].a);
      s.wb[q] = ld_status(&st.lvl0[i].b);
    }
  }
  if (!s.r1) {
    s.w1a = ld_status(&st.lvl1[s.blk1 * kFan + lane].a);
    s.w1b = ld_status(&st.lvl1[s.blk1 * kFan + lane].b);
  }
  if (!s.r2) {
    s.w2a = ld_status(&st.lvl2[lane].a);
    s.w2b = ld_status(&st.lvl2[lane].b);
  }
}

__device__ __forceinline__ void lb_check(LookBack &s, uint32_t epoch) {
#pragma unroll
  for (int q = 0; q < kRecent; ++q)
    s.r[q] = s.r[q] || (word_ready(s.wa[q], epoch) && word_ready(s.wb[q], epoch));
  s.r1 = s.r1 || (word_ready(s.w1a, epoch) && word_ready(s.w1b, epoch));
  s.r2 = s.r2 || (word_ready(s.w2a, epoch) && word_ready(s.w2b, epoch));
}

// Words lb_done waits for: all of them, or only those a tile that closes a
// superblock (block: also closes a block) needs for the aggregates it
// publishes (see publish_higher).
enum class Need { kAll, kSuperblock, kBlock };

__device__ __forceinline__ bool lb_done(const LookBack &s, Need need = Need::kAll) {
  bool pending = false;
  if (need == Need::kAll) pending = __ballot(!s.r2) != 0;
  if (need != Need::kSuperblock) pending = pending || __ballot(!s.r1) != 0;
#pragma unroll
  for (int q = 0; q < kRecent; ++q)
    if (need != Need::kSuperblock || q == s.nw - 1) pending = pending || __ballot(!s.r[q]) != 0;
  return !pending;
}

// Entries of recent window q.
__device__ __forceinline__ int window_count(const LookBack &s, int q) {
  return q < s.nw - 1 ? kFan : (q == s.nw - 1 ? s.n0 : 0);
}

// Window q of the look-back in sequence order, q = -2 (level 2), -1 (level
// 1), 0 .. kRecent - 1 (recent level-0 windows), as this lane's map and the
// window's entry count; selected, not indexed, so the words stay in
// registers. For the rolled loops of the rare careful paths.
__device__ __forceinline__ Map window_word(const LookBack &s, int q, int &count) {
  uint64_t wa = s.w2a, wb = s.w2b;
  count = s.n2;
  if (q == -1) {
    wa = s.w1a;
    wb = s.w1b;
    count = s.n1;
  }
#pragma unroll
  for (int k = 0; k < kRecent; ++k) {
    if (q == k) {
      wa = s.wa[k];
      wb = s.wb[k];
      count = window_count(s, k);
    }
  }
  return word_map(wa, wb);
}

// The tile's incoming value: h0 pushed through the complete windows in
// sequence order (level 2, level 1, then the recent level-0 windows; fixed
// shapes, so the result depends only on the words and the tile index).
// Plain products, which agree with the careful rule whenever h0 and every
// word are finite: a head's multiplier is exactly zero, so a plain product
// also drops what precedes it, and a multiplier that underflowed to zero
// instead of to the smallest subnormal changes a finite value by at most
// 2^-149 of the value it multiplies.
__device__ __forceinline__ float lb_value(const LookBack &s, float h0, int lane) {
  using P = AffOp<false, false>;
  float v = P::apply(window_total(word_map(s.w2a, s.w2b), s.n2, lane), h0);
  v = P::apply(window_total(word_map(s.w1a, s.w1b), s.n1, lane), v);
#pragma unroll
  for (int q = 0; q < kRecent; ++q) {
    const int count = window_count(s, q);
    if (count > 0) v = P::apply(window_total(word_map(s.wa[q], s.wb[q]), count, lane), v);
  }
  return v;
}

// The same by Op's rule (window totals by window_total_careful, heads
// honoured), one window at a time.
template <class Op>
__device__ __forceinline__ float lb_value_careful(const LookBack &s, float h0, int lane) {
  float v = h0;
#pragma unroll 1
  for (int q = -2; q < kRecent; ++q) {
    int count;
    const Map m = window_word(s, q, count);
    if (count > 0) v = Op::apply(window_total_careful<Op>(m, count, lane), v);
  }
  return v;
}

// Plain, or careful when the plain value is an inf or NaN: a non-finite h0 or
// word always leaves it so (no IEEE step of a plain window total or of
// applying it to a value turns a non-finite value finite again), and the
// careful rule can differ only then.
template <class Op>
__device__ __forceinline__ float lb_finish(const LookBack &s, float h0, int lane) {
  const float v = lb_value(s, h0, lane);
  if (__builtin_expect(!uniform_nonfinite(v), 1)) return v;
  return lb_value_careful<Op>(s, h0, lane);
}

// The last tile of a superblock publishes the superblock's aggregate (level
// 1): its own superblock's level-0 window composed with its own aggregate.
// The last tile of a block also publishes the block's aggregate (level 2):
// the level-1 window of its block and its recent level-0 windows before its
// superblock, composed with the superblock's aggregate. Neither needs any
// word from before the block, so both are published before the tile's
// level-2 words arrive; every aggregate is thus a fixed-depth function of
// level-0 words and no chain of look-backs runs through the higher levels.
// Careful rule throughout: a later look-back may push an inf through these
// multipliers.
template <class Op>
__device__ __forceinline__ void publish_higher(const LinearStatus &st, int64_t tile,
                                               const LookBack &s, const Map &own,
                                               uint32_t epoch, int lane) {
  const int64_t sb = tile / kFan;
  const int64_t blk = sb / kFan;
  const bool closes_block = sb - blk * kFan == kFan - 1;
  // Windows -1 .. nw - 2 (the block's level-1 window and the whole recent
  // superblocks) go into PB, which only the last tile of a block needs;
  // window nw - 1 (the own superblock up to the tile) is P0.
  Map pb = identity_map(), sbm = own;
#pragma unroll 1
  for (int q = closes_block ? -1 : s.nw - 1; q < s.nw; ++q) {
    int count;
    const Map t = window_total_careful<Op>(window_word(s, q, count), count, lane);
    if (q == s.nw - 1)
      sbm = Op::compose(t, own);
    else
      pb = Op::compose(pb, t);
  }
  if (lane == 0) {
    st_map(st.lvl1[sb], epoch, sbm);
    if (closes_block) st_map(st.lvl2[blk], epoch, Op::compose(pb, sbm));
  }
}

// Independent sequences inside one scan (the batched form): `len` elements
// each, sequence k starting from h0[k] (0 if h0 is null) and, when h_last is
// not null, leaving its last value in h_last[k]. len == 0: one sequence.
// i / len is evaluated as (t1 + ((i - t1) >> sh1)) >> sh2 with
// t1 = mulhi(magic, i), the round-up method for division by an invariant
// integer (Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994), exact for every 32-bit i.
struct Segments {
  const float *h0;
  float *h_last;
  uint32_t len, magic, sh1, sh2;
};

// Position t of element i within its sequence, and the sequence's index k
// (i < 2^32; len >= 1).
__device__ __forceinline__ void seg_pos(uint32_t i, const Segments &sg, uint32_t &k,
                                        uint32_t &t) {
  const uint32_t t1 = __umulhi(sg.magic, i);
  k = (t1 + ((i - t1) >> sg.sh1)) >> sg.sh2;
  t = i - k * sg.len;
}

// Whether the 4 elements from i on hold the first or the last element of a
// sequence (then each is looked at separately).
__device__ __forceinline__ bool seg_edge(uint32_t i, const Segments &sg) {
  uint32_t k, t;
  seg_pos(i, sg, k, t);
  return t == 0 || t + 4 >= sg.len;
}

// Bit j set when element i + j (j < 4, below n) is the first of a sequence.
__device__ __forceinline__ uint32_t seg_heads(int64_t i, int64_t n, const Segments &sg) {
  uint32_t bits = 0;
  if (i < n && seg_edge(uint32_t(i), sg)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (i + j < n) {
        uint32_t k, t;
        seg_pos(uint32_t(i + j), sg, k, t);
        if (t == 0) bits |= 1u << j;
      }
    }
  }
  return bits;
}

// Loads one tile (rows of float4 per wave); past n the identity map (1, 0).
// With segments, the first element of every sequence has its b replaced by
// a*h0 + b (its value, whatever precedes it) and its multiplier set to zero;
// hd is non-zero if the lane holds a head.
template <bool Seg>
__device__ __forceinline__ void load_tile(const float *__restrict__ a,
                                          const float *__restrict__ b, int64_t n, int64_t tile,
                                          const Segments &sg, float4 (&va)[Shape<Seg>::kRows],
                                          float4 (&vb)[Shape<Seg>::kRows],
                                          uint32_t &hd) {
  constexpr int kRows = Shape<Seg>::kRows, kWaveElems = Shape<Seg>::kWaveElems,
                kTileElems = Shape<Seg>::kTileElems;
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
  hd = 0u;
  if constexpr (Seg) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t off = wave_start + r * kRowElems + lane * 4;
      const uint32_t bits = seg_heads(off, n, sg);
      hd |= bits;
      if (bits) {
        float ta[4] = {va[r].x, va[r].y, va[r].z, va[r].w};
        float tb[4] = {vb[r].x, vb[r].y, vb[r].z, vb[r].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((bits >> j) & 1u) {
            uint32_t k, t;
            seg_pos(uint32_t(off + j), sg, k, t);
            tb[j] = __builtin_fmaf(ta[j], sg.h0 ? sg.h0[k] : 0.0f, tb[j]);
            ta[j] = 0.0f;
          }
        }
        va[r] = make_float4(ta[0], ta[1], ta[2], ta[3]);
        vb[r] = make_float4(tb[0], tb[1], tb[2], tb[3]);
      }
    }
  }
}

// Data waves, phase 1: the lane's 4 items composed, a wave scan per row (im:
// the lane's inclusive prefix within its row) and the wave's aggregate (rows
// folded in order), returned in every lane. Plain products; a multiplier
// that underflowed to zero is nudged where it is used later (im and the row
// totals) unless the lanes it covers hold an exact zero multiplier, so the
// results stay right when an infinite carry arrives later. Returns true if
// the wave holds an inf or NaN (then a plain product may have formed 0 * inf
// and an offset may have met an underflowed zero, and an infinite multiplier
// is no affine map at all): the tile is then evaluated in sequence instead
// (seq_tile) and these results are not used.
// Sequence heads (batched scans) need no rule of their own here: a head's
// multiplier is exactly zero, so with finite values a plain product already
// drops what precedes it. Only the wave aggregate carries a head bit (set if
// the wave holds a head), for the careful compositions downstream, and
// tile_apply honours heads itself when the incoming value is not finite.
template <bool Seg, int kRows>
__device__ __forceinline__ bool tile_local_scan(const float4 (&va)[kRows],
                                                const float4 (&vb)[kRows],
                                                uint32_t hd, Map (&im)[kRows], Map &wagg) {
  using Op = AffOp<false, false>;
  using COp = AffOp<false, true>;
  const int lane = threadIdx.x & 63;
  bool bad = false;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    Map m = Map{va[r].x, vb[r].x, 0u};
    m = Op::compose(m, Map{va[r].y, vb[r].y, 0u});
    m = Op::compose(m, Map{va[r].z, vb[r].z, 0u});
    m = Op::compose(m, Map{va[r].w, vb[r].w, 0u});
    wave_scan<Op>(m);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(m.a == 0.0f) != 0, 0)) {  // an underflow or a zero
      const float z = fminf(fminf(fabsf(va[r].x), fabsf(va[r].y)),
                            fminf(fabsf(va[r].z), fabsf(va[r].w)));
      const uint64_t zeros = __builtin_amdgcn_ballot_w64(z == 0.0f);
      const uint64_t upto = ~uint64_t(0) >> (63 - lane);  // lanes 0 .. lane
      if (m.a == 0.0f && (zeros & upto) == 0) m.a = nudge(m.a);
    }
    im[r] = m;
  }
  // An inf or NaN anywhere in a row leaves the row's total non-finite (no
  // IEEE operation of a plain composition turns it finite again).
  wagg = lane_map(im[0], 63);
  bad = bad || uniform_nonfinite(wagg.a) || uniform_nonfinite(wagg.b);
#pragma unroll
  for (int r = 1; r < kRows; ++r) {
    const Map t = lane_map(im[r], 63);
    bad = bad || uniform_nonfinite(t.a) || uniform_nonfinite(t.b);
    wagg = COp::compose(wagg, t);
  }
  if constexpr (Seg) wagg.head = __builtin_amdgcn_ballot_w64(hd != 0u) != 0 ? 1u : 0u;
  return bad;
}

// Data waves, phase 2: carry into each row, then into each lane's chunk, then
// re-run the recurrence over the lane's 4 items and store (with segments,
// the last value of each sequence also goes to h_last).
template <bool Seg, int kRows = Shape<Seg>::kRows>
__device__ __forceinline__ void tile_apply(const float4 (&va)[kRows], const float4 (&vb)[kRows],
                                           const Map (&im)[kRows], float c,
                                           float *__restrict__ h, int64_t n, int64_t tile,
                                           const Segments &sg) {
  constexpr int kWaveElems = Shape<Seg>::kWaveElems, kTileElems = Shape<Seg>::kTileElems;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t wave_start = tile * kTileElems + int64_t(wave) * kWaveElems;
  const bool full = (tile + 1) * kTileElems <= n;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int64_t off = wave_start + r * kRowElems + lane * 4;
    // A head's multiplier is exactly zero, so while the values are finite
    // the plain recurrence already ignores what precedes a head.
    const float end = __builtin_fmaf(im[r].a, c, im[r].b);  // h after this lane's chunk
    const float cin = dpp<kWaveShr1, 0xf, 0xf>(c, end);     // h before it
    float4 o;
    o.x = __builtin_fmaf(va[r].x, cin, vb[r].x);
    o.y = __builtin_fmaf(va[r].y, o.x, vb[r].y);
    o.z = __builtin_fmaf(va[r].z, o.y, vb[r].z);
    o.w = __builtin_fmaf(va[r].w, o.z, vb[r].w);
    if constexpr (Seg) {
      // An inf or NaN carry (from an earlier sequence: the tile's own values
      // are finite) must not reach past a head: a lane whose prefix holds a
      // head takes the prefix's offset, and a head item takes its own.
      if (__builtin_expect(uniform_nonfinite(c), 0)) {
        const uint32_t hb = seg_heads(off, n, sg);
        const uint64_t heads = __builtin_amdgcn_ballot_w64(hb != 0u);
        const uint64_t upto = ~uint64_t(0) >> (63 - lane);
        const float e = (heads & upto) ? im[r].b : end;
        const float ci = dpp<kWaveShr1, 0xf, 0xf>(c, e);
        o.x = (hb & 1u) ? vb[r].x : __builtin_fmaf(va[r].x, ci, vb[r].x);
        o.y = (hb & 2u) ? vb[r].y : __builtin_fmaf(va[r].y, o.x, vb[r].y);
        o.z = (hb & 4u) ? vb[r].z : __builtin_fmaf(va[r].z, o.y, vb[r].z);
        o.w = (hb & 8u) ? vb[r].w : __builtin_fmaf(va[r].w, o.z, vb[r].w);
        c = lane_f(e, 63);
      } else {
        c = lane_f(end, 63);
      }
    } else {
      c = lane_f(end, 63);
    }
    if (full) {
      store_nt(h + off, o);
    } else {
      const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (off + j < n) h[off + j] = ov[j];
    }
    if constexpr (Seg) {
      if (sg.h_last && off < n && seg_edge(uint32_t(off), sg)) {
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (off + j < n) {
            uint32_t k, t;
            seg_pos(uint32_t(off + j), sg, k, t);
            if (t == sg.len - 1) sg.h_last[k] = ov[j];
          }
        }
      }
    }
  }
}

// One claim on the launch's claims word, ((epoch - 1) << 32) | claims made so
// far: the claimed tile (ntiles or more means none) and the launch's epoch.
// Every workgroup claims one tile at a time until its first failed claim, so
// a launch makes exactly ntiles + gridDim.x claims; the last of them hands
// the next epoch (count 0) to the next launch on the workspace.
struct Claim {
  int64_t tile;
  uint32_t epoch;
};
__device__ __forceinline__ Claim claim_tile(const LinearStatus &st, int64_t ntiles, int lane) {
  unsigned long long w = 0;
  if (lane == 0) {
    w = __hip_atomic_fetch_add(st.claims, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (uint32_t(w) == uint32_t(ntiles) + gridDim.x - 1u) {
      const uint32_t hi = uint32_t(w >> 32);
      const uint32_t next = hi + 1u >= st.epoch_cycle ? 0u : hi + 1u;
      __hip_atomic_store(st.claims, (unsigned long long)next << 32, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const uint32_t count = __builtin_amdgcn_readfirstlane(uint32_t(w));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(w >> 32));
  return {count < ntiles ? int64_t(count) : ntiles, hi + 1u};
}

// The tile a workgroup scans after tile t (t < 0: its first), claimed anew;
// ntiles means none, and a workgroup claims nothing after a failed claim.
__device__ __forceinline__ int64_t successor(int64_t t, int64_t ntiles, const LinearStatus &st,
                                             int lane) {
  if (t >= ntiles) return ntiles;
  return claim_tile(st, ntiles, lane).tile;
}

// Called by every wave as it finishes. Epochs are 31-bit, so after a full
// cycle a status word left from the previous pass over the epochs could look
// current; the launch that takes the cycle's last epoch therefore counts its
// waves out (acquire-release, so every status access of the launch comes
// before), and the last wave out clears every status word (epoch 0, never
// current) for the next cycle.
__device__ __forceinline__ void check_out(const LinearStatus &st, uint32_t epoch, int lane) {
  if (epoch < st.epoch_cycle) return;
  unsigned long long *done = st.claims + LinearStatus::kDoneOffset;
  unsigned long long d = 0;
  if (lane == 0)
    d = __hip_atomic_fetch_add(done, 1ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t waves = uint32_t(gridDim.x) * (blockDim.x / 64u);
  if (__builtin_amdgcn_readfirstlane(uint32_t(d)) != waves - 1u) return;
  uint64_t *words = reinterpret_cast<uint64_t *>(st.lvl0);  // the levels lie back to back
  for (int64_t i = lane; i < st.nwords; i += 64)
    __hip_atomic_store(words + i, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (lane == 0) __hip_atomic_store(done, 0ull, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS shared by the waves of one workgroup. Per-tile values are kept in
// 4-entry rings indexed by the tile's position j in the workgroup's sequence
// (j % 4): a tile's entries are written two iterations before the last read,
// and every hand-over crosses a barrier. The parked a/b of two tiles wait
// there for their look-backs (slot j % 2; each wave reads back only what it
// wrote itself).
template <bool Seg>
struct Shared {
  static constexpr int kWaves = Shape<Seg>::kWaves, kRows = Shape<Seg>::kRows;
  float4 park[2][kWaves][kRows][2][64];  // a, b rows of two parked tiles
  Map wave[4][kWaves];                   // per-wave aggregates
  float2 wpre[4][kWaves];                // their inclusive prefixes (plain products)
  Map tile[4];                           // tile aggregates
  uint32_t wave_seq[4][kWaves];          // the wave's rows hold an inf or NaN
  uint32_t tile_seq[4];                  // so does the tile: evaluated in sequence (seq_tile)
  float carry[4][kWaves];                // h entering each wave's rows
  int64_t ids[4];                        // claimed tiles, in claim order
  unsigned arrived[2];                   // data waves done with a tile's local scan
  uint32_t epoch;                        // this launch's epoch
};

template <bool Seg, int kRows = Shape<Seg>::kRows>
__device__ __forceinline__ void park(Shared<Seg> &sh, int slot, const float4 (&va)[kRows],
                                     const float4 (&vb)[kRows]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    sh.park[slot][wave][r][0][lane] = va[r];
    sh.park[slot][wave][r][1][lane] = vb[r];
  }
}
template <bool Seg, int kRows = Shape<Seg>::kRows>
__device__ __forceinline__ void unpark(const Shared<Seg> &sh, int slot, float4 (&va)[kRows],
                                       float4 (&vb)[kRows]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    va[r] = sh.park[slot][wave][r][0][lane];
    vb[r] = sh.park[slot][wave][r][1][lane];
  }
}

// A tile holding an inf or NaN is evaluated element by element, in sequence
// order, from its exact incoming value h_in, by one lane of the control wave
// from the a/b parked in LDS: that gives the sequential loop's IEEE results
// exactly. A parallel scan cannot in general: it multiplies multipliers, and
// a multiplier of +-inf makes the state after it depend on the sign of the
// state before it, which no affine map of the incoming value expresses (a
// composition forms inf*x + inf*y where the loop forms inf*(x + y)). The
// function writes the tile's outputs (and, with segments, h_last) and
// returns the value after the tile's last element; the tile is then
// published as a constant map (a head) with that value, so later tiles see
// exactly the loop's state. Only inputs holding inf or NaN take this path.
template <bool Seg>
__device__ __forceinline__ float seq_tile(const Shared<Seg> &sh, int slot, int64_t tile, float h_in,
                          float *__restrict__ h, int64_t n, const Segments &sg) {
  constexpr int kWaves = Shape<Seg>::kWaves, kRows = Shape<Seg>::kRows,
                kTileElems = Shape<Seg>::kTileElems;
  float v = h_in;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll 1
    for (int w = 0; w < kWaves; ++w)
#pragma unroll 1
      for (int r = 0; r < kRows; ++r)
#pragma unroll 1
        for (int l = 0; l < 64; ++l) {
          const float4 av = sh.park[slot][w][r][0][l], bv = sh.park[slot][w][r][1][l];
          const float ta[4] = {av.x, av.y, av.z, av.w}, tb[4] = {bv.x, bv.y, bv.z, bv.w};
          const int64_t off = tile * kTileElems + int64_t(w) * Shape<Seg>::kWaveElems +
                              r * kRowElems + l * 4;
          for (int j = 0; j < 4; ++j) {
            if (off + j >= n) continue;
            bool head = false;
            uint32_t k = 0, t = 1;
            if constexpr (Seg) {
              seg_pos(uint32_t(off + j), sg, k, t);
              head = t == 0;
            }
            v = head ? tb[j] : __builtin_fmaf(ta[j], v, tb[j]);
            h[off + j] = v;
            if constexpr (Seg) {
              if (sg.h_last && t == sg.len - 1) sg.h_last[k] = v;
            }
          }
        }
  }
  return lane_f(v, 0);
}

// Data waves: local scan of a loaded tile; the last data wave to finish folds
// the wave aggregates into the tile aggregate and publishes it (level 0) at
// once, without waiting for any other workgroup.
template <bool Seg, int kRows = Shape<Seg>::kRows>
__device__ __forceinline__ void scan_and_publish(const float4 (&va)[kRows],
                                                 const float4 (&vb)[kRows],
                                                 uint32_t hd, Map (&im)[kRows],
                                                 Shared<Seg> &sh, int ring, int slot,
                                                 const LinearStatus &st, int64_t tile,
                                                 uint32_t epoch) {
  constexpr int kWaves = Shape<Seg>::kWaves;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  Map wagg;
  const uint32_t seq = tile_local_scan<Seg, kRows>(va, vb, hd, im, wagg) ? 1u : 0u;
  if (lane == 0) {
    sh.wave[ring][wave] = wagg;
    sh.wave_seq[ring][wave] = seq;
  }
  unsigned prior = 0;
  if (lane == 0)
    prior = __hip_atomic_fetch_add(&sh.arrived[slot], 1u, __ATOMIC_ACQ_REL,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
  prior = __builtin_amdgcn_readfirstlane(prior);
  if (prior == kWaves - 1) {
    // The fold is on the path to the tile's publication: one LDS round trip
    // (lane w reads wave w's aggregate) and a DPP scan. Plain products give
    // the careful rule's map when every wave aggregate is finite (the only
    // case in which it is published): a head's multiplier is exactly zero,
    // and an underflow is nudged at the end unless a wave's multiplier is
    // exactly zero. The inclusive prefixes go to LDS for the carries.
    Map x = identity_map();
    uint32_t sq = 0u;
    if (lane < kWaves) {
      x = sh.wave[ring][lane];
      sq = sh.wave_seq[ring][lane];
    }
    const bool zero = __builtin_amdgcn_ballot_w64(x.a == 0.0f) != 0;
    const uint32_t head = __builtin_amdgcn_ballot_w64(x.head != 0u) != 0 ? 1u : 0u;
    const uint32_t tseq = __builtin_amdgcn_ballot_w64(sq != 0u) != 0 ? 1u : 0u;
    wave_scan<AffOp<false, false>>(x);
    if (lane < kWaves) sh.wpre[ring][lane] = make_float2(x.a, x.b);
    Map g = lane_map(x, kWaves - 1);
    if (g.a == 0.0f && !zero) g.a = nudge(g.a);
    g.head = head;
    if (lane == 0) {
      // A tile evaluated in sequence is published by the control wave once
      // it has its value (see seq_tile).
      if (!tseq) st_map(st.lvl0[tile], epoch, g);
      sh.tile[ring] = g;
      sh.tile_seq[ring] = tseq;
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
// A workgroup's tiles t_0, t_1, ... move through a pipeline, one stage per
// iteration; in iteration j, between barriers C_{j-1} and C_j:
//   data waves   - issue the loads of t_{j+2} (wave 0 first claims t_{j+3}),
//                  scan t_{j+1} (loaded one iteration earlier) and publish its
//                  level-0 aggregate; after C_j, apply t_{j-1}'s carries to
//                  its parked a/b, store it, and park t_{j+1}'s a/b in the
//                  slot t_{j-1} left;
//   control wave - issues the first status reads of t_j's look-back together
//                  with the next reads of t_{j-1}'s, finishes t_{j-1}'s
//                  look-back, publishes its higher-level aggregates if it is
//                  the last tile of a superblock or block, and leaves the
//                  carries of its waves in LDS.
// So a tile's loads have an iteration to arrive, its look-back starts an
// iteration after its predecessors were published and has an iteration and
// a half to finish, and the control wave's status reads never queue behind
// data loads (the vector memory counter retires in order). The claim atomic
// is issued ahead of the loads it must not wait for, and its result is read
// one barrier later. At the start the control wave's first three claims are
// dependent atomics on a counter every workgroup is hitting at once, so each
// is followed by a barrier (A0, A1, A) after which the data waves start
// loading the tile just claimed, rather than all three waiting for the last
// claim (measured: 2 us of 273 per launch at 2^27 elements).
//
// Every wait is for something a lower tile produces before it waits on
// anything itself (level-0 aggregates right after its local scan, higher
// levels after the look-back of a lower tile), and a workgroup only waits on
// tiles lower than the ones it owns; so the lowest unfinished tile can always
// finish, however many workgroups the device keeps resident.
// The launch's epoch arrives with every claim (see claim_tile), so a launch
// recorded in a HIP graph gets a fresh epoch on every replay.
template <bool Seg>
__global__ __launch_bounds__(Shape<Seg>::kThreads + 64) void linear_scan_kernel(
    const float *__restrict__ a, const float *__restrict__ b, float h0,
    float *__restrict__ h, int64_t n, int64_t ntiles, LinearStatus st, Segments sg) {
  using COp = AffOp<Seg, true>;
  // The control wave's compositions honour heads in both forms: a tile with
  // an infinite multiplier is published as one (see seq_tile).
  using HOp = AffOp<true, true>;
  constexpr int kWaves = Shape<Seg>::kWaves, kRows = Shape<Seg>::kRows;
  __shared__ Shared<Seg> sh;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (wave == kWaves) {
    const Claim first = claim_tile(st, ntiles, lane);
    const uint32_t epoch = first.epoch;
    const int64_t t0 = first.tile;
    if (lane == 0) {
      sh.ids[0] = t0;
      sh.epoch = epoch;
    }
    __syncthreads();  // A0: the first tile and the epoch visible
    const int64_t t1 = successor(t0, ntiles, st, lane);
    if (lane == 0) sh.ids[1] = t1;
    __syncthreads();  // A1: the second tile visible
    const int64_t t2 = successor(t1, ntiles, st, lane);
    if (lane == 0) {
      sh.ids[2] = t2;
      sh.arrived[0] = 0;
      sh.arrived[1] = 0;
    }
    __syncthreads();  // A: the third claim visible
    __syncthreads();  // B: t_0 scanned and published
    // Look-backs of t_{j-1} (lp) and t_j (ln). t_j's first status reads are
    // issued at the end of iteration j and read at the start of iteration j+1,
    // so their round trip overlaps the barrier and the data waves' work. The
    // two LookBack variables swap roles every iteration (the loop is unrolled
    // by two) rather than being copied, since a copy would wait for the reads.
    LookBack l0, l1;
    int64_t tp = ntiles;
    int j = 0;
    auto step = [&](LookBack &lp, LookBack &ln) {
      const int64_t tn = sh.ids[j & 3];  // claimed before barrier C of iteration j-3
      if (tp < ntiles) {
        const int rp = (j - 1) & 3;
        const bool seq = sh.tile_seq[rp] != 0;  // rare: an inf or NaN in the tile
        // Prefix of the waves before this lane's wave (read before the wait).
        const float2 pre = lane > 0 && lane < kWaves ? sh.wpre[rp][lane - 1] : make_float2(1.0f, 0.0f);
        const int64_t sb = tp / kFan;
        // A tile that closes a superblock publishes as soon as the words its
        // aggregates need are complete (before the rest, unless it is
        // evaluated in sequence: then its own aggregate is its final value).
        // One call site each for lb_finish and publish_higher.
        bool publish = tp - sb * kFan == kFan - 1;
        Need need = Need::kAll;
        if (publish && !seq)
          need = (sb & (kFan - 1)) == kFan - 1 ? Need::kBlock : Need::kSuperblock;
        Map own = sh.tile[rp];
        float h_in = 0.0f;
        lb_check(lp, epoch);
        for (;;) {
          while (!lb_done(lp, need)) {
            __builtin_amdgcn_s_sleep(1);
            lb_issue(lp, st, lane);
            lb_check(lp, epoch);
          }
          if (need == Need::kAll) {
            h_in = lb_finish<HOp>(lp, h0, lane);
            if (__builtin_expect(seq, 0)) {
              own = Map{0.0f, seq_tile<Seg>(sh, (j - 1) & 1, tp, h_in, h, n, sg), 1u};
              if (lane == 0) st_map(st.lvl0[tp], epoch, own);
            }
          }
          if (publish) publish_higher<HOp>(st, tp, lp, own, epoch, lane);
          publish = false;
          if (need == Need::kAll) break;
          need = Need::kAll;
        }
        if (!seq) {
          // The waves' aggregates are finite: with a finite h_in, the plain
          // prefix of the waves before wave w applied to h_in gives the
          // careful rule's value (a head's multiplier is exactly zero).
          if (__builtin_expect(!uniform_nonfinite(h_in), 1)) {
            if (lane < kWaves)
              sh.carry[rp][lane] = lane == 0 ? h_in : __builtin_fmaf(pre.x, h_in, pre.y);
          } else if (lane == 0) {
            float c = h_in;
            for (int w = 0; w < kWaves; ++w) {
              sh.carry[rp][w] = c;
              c = COp::apply(sh.wave[rp][w], c);
            }
          }
        }
      }
      if (tn < ntiles) {
        lb_init(ln, tn, lane);
        lb_issue(ln, st, lane);
      }
      tp = tn;
      __syncthreads();  // C_j: carries of t_{j-1}; t_{j+1} published; t_{j+3} claimed
      ++j;
    };
    for (;;) {
      step(l0, l1);
      if (tp >= ntiles) break;
      step(l1, l0);
      if (tp >= ntiles) break;
    }
    check_out(st, epoch, lane);
    return;
  }

  __syncthreads();  // A0
  const uint32_t epoch = sh.epoch;
  int64_t tp = ntiles, t0 = sh.ids[0];
  // Register stages: (va, vb) tile being applied, (na, nb) tile being
  // scanned, (ma, mb) tile being loaded; prefixes of the two parked tiles.
  float4 va[kRows], vb[kRows], na[kRows], nb[kRows];
  uint32_t hv, hn;
  Map imp[kRows], imw[kRows];
  if (t0 < ntiles) load_tile<Seg>(a, b, n, t0, sg, va, vb, hv);
  __syncthreads();  // A1
  int64_t t1 = sh.ids[1];
  if (t1 < ntiles) load_tile<Seg>(a, b, n, t1, sg, na, nb, hn);
  __syncthreads();  // A
  int64_t t2 = sh.ids[2];
  if (t0 < ntiles) {
    scan_and_publish<Seg>(va, vb, hv, imw, sh, 0, 0, st, t0, epoch);
    park(sh, 0, va, vb);
  }
  __syncthreads();  // B
  // In iteration j: tp = t_{j-1}, t0 = t_j, t1 = t_{j+1}, t2 = t_{j+2}.
  for (int j = 0; j == 0 || tp < ntiles; ++j) {
    int64_t claimed = ntiles;
    if (wave == 0 && t2 < ntiles) claimed = successor(t2, ntiles, st, lane);
    float4 ma[kRows], mb[kRows];
    uint32_t hm;
    if (t2 < ntiles) load_tile<Seg>(a, b, n, t2, sg, ma, mb, hm);
    Map nim[kRows];
    if (t1 < ntiles)
      scan_and_publish<Seg>(na, nb, hn, nim, sh, (j + 1) & 3, (j + 1) & 1, st, t1, epoch);
    if (wave == 0 && lane == 0) sh.ids[(j + 3) & 3] = claimed;
    __syncthreads();  // C_j
    if (tp < ntiles && __builtin_expect(sh.tile_seq[(j - 1) & 3] == 0, 1)) {  // else the control wave wrote it
      unpark(sh, (j + 1) & 1, va, vb);  // t_{j-1} sits in slot (j - 1) % 2
      tile_apply<Seg>(va, vb, imp, sh.carry[(j - 1) & 3][wave], h, n, tp, sg);
    }
    if (t1 < ntiles) park(sh, (j + 1) & 1, na, nb);
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      imp[r] = imw[r];
      imw[r] = nim[r];
      na[r] = ma[r];
      nb[r] = mb[r];
    }
    hn = hm;
    tp = t0;
    t0 = t1;
    t1 = t2;
    t2 = sh.ids[(j + 3) & 3];
  }
  check_out(st, epoch, lane);
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

// Status memory of the allocation-free entry point: file-scope device memory,
// one copy per GPU, sized for the largest launch (kLinearMaxTiles tiles,
// 2^31 elements) in the workspace layout (claims word and done count, then
// the three levels, each 256-byte aligned). It starts zeroed when the code
// object is loaded: epoch 0 everywhere and the claims word at epoch 1 with
// nothing claimed, which is the state every launch leaves for the next, so
// it is never cleared again. In host code its name is not a device address:
// linear_noalloc_status takes the address from hipGetSymbolAddress.
constexpr size_t pad256(size_t x) { return (x + 255) / 256 * 256; }
constexpr size_t kNoAllocLvl0 = pad256(size_t(kLinearMaxTiles) * sizeof(AggWord));
constexpr size_t kNoAllocLvl1 = pad256(size_t(kLinearMaxTiles / 64) * sizeof(AggWord));
constexpr size_t kNoAllocLvl2 = pad256(size_t(kLinearMaxTiles / 4096) * sizeof(AggWord));
constexpr size_t kNoAllocBytes = 256 + kNoAllocLvl0 + kNoAllocLvl1 + kNoAllocLvl2;
__device__ __align__(256) unsigned char scratch[kNoAllocBytes];

}  // namespace

size_t linear_noalloc_bytes() { return kNoAllocBytes; }

int linear_noalloc_status(LinearStatus *status, uint32_t epoch_cycle) {
  constexpr int kMaxDevices = 64;
  static void *ptrs[kMaxDevices];  // per device: scratch's address there
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= kMaxDevices) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
      void *p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return 0;
      ptrs[dev] = p;
    }
  }
  char *base = static_cast<char *>(ptrs[dev]);
  status->claims = reinterpret_cast<unsigned long long *>(base);
  status->lvl0 = reinterpret_cast<AggWord *>(base + 256);
  status->lvl1 = reinterpret_cast<AggWord *>(base + 256 + kNoAllocLvl0);
  status->lvl2 = reinterpret_cast<AggWord *>(base + 256 + kNoAllocLvl0 + kNoAllocLvl1);
  status->nwords = int64_t((kNoAllocBytes - 256) / sizeof(uint64_t));
  status->epoch_cycle = epoch_cycle;
  return 1;
}

int64_t linear_tile_elems(bool segmented) {
  return segmented ? Shape<true>::kTileElems : Shape<false>::kTileElems;
}

hipError_t launch_linear_scan(const float *a, const float *b, float h0, float *h,
                              int64_t n, int64_t ntiles, LinearStatus status,
                              int resident_wgs, const float *seg_h0, float *seg_h_last,
                              uint32_t seg_len, hipStream_t stream) {
  const unsigned grid = unsigned(ntiles < resident_wgs ? ntiles : resident_wgs);
  Segments sg{seg_h0, seg_h_last, seg_len, 0, 0, 0};
  if (seg_len > 0) {  // magic number for division by seg_len (see Segments)
    uint32_t l = 0;
    while ((uint64_t(1) << l) < seg_len) ++l;
    sg.magic = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - seg_len)) / seg_len + 1);
    sg.sh1 = l < 1 ? l : 1;
    sg.sh2 = l > 0 ? l - 1 : 0;
  }
  if (seg_len == 0)
    hipLaunchKernelGGL(linear_scan_kernel<false>, dim3(grid), dim3(Shape<false>::kThreads + 64), 0,
                       stream, a,
                       b, h0, h, n, ntiles, status, sg);
  else
    hipLaunchKernelGGL(linear_scan_kernel<true>, dim3(grid), dim3(Shape<true>::kThreads + 64), 0,
                       stream, a,
                       b, h0, h, n, ntiles, status, sg);
  return hipGetLastError();
}

int linear_wgs_per_cu() {
  int plain = 0, seg = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &plain, reinterpret_cast<const void *>(linear_scan_kernel<false>),
          Shape<false>::kThreads + 64, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &seg, reinterpret_cast<const void *>(linear_scan_kernel<true>),
          Shape<true>::kThreads + 64, 0) !=
          hipSuccess)
    return 0;
  return plain < seg ? plain : seg;
}

// h = a * b elementwise: the linear scan's HBM traffic (two streams read,
// one written) with no dependence between elements, as the attainable-rate
// reference for the scan. One 16-byte vector per lane and one block of 256
// vectors per workgroup: of the shapes measured for this traffic on gfx950
// (grid-stride loops of 1024 to 16384 workgroups, persistent workgroups with
// a tile in flight, 1 to 8 vectors per lane, 256 to 1024 lanes per
// workgroup) the many short workgroups were fastest. The lane after the last
// whole vector takes the 0 to 3 elements left.
__global__ __launch_bounds__(256) void stream_mul_kernel(const float *__restrict__ a,
                                                         const float *__restrict__ b,
                                                         float *__restrict__ h, int64_t n) {
  const int64_t nvec = n / 4;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < nvec) {
    const float4 x = load_nt(a + 4 * i), y = load_nt(b + 4 * i);
    store_nt(h + 4 * i, make_float4(x.x * y.x, x.y * y.y, x.z * y.z, x.w * y.w));
  } else if (i == nvec) {
    for (int64_t k = 4 * nvec; k < n; ++k) h[k] = a[k] * b[k];
  }
}

hipError_t launch_stream_mul_f32(const float *a, const float *b, float *h, int64_t n,
                                 hipStream_t stream) {
  const int64_t blocks = (n / 4 + 1 + 255) / 256;  // the vectors and the tail lane
  hipLaunchKernelGGL(stream_mul_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, a, b, h,
                     n);
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
