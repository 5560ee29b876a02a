// C-ABI entry points of libssmscan: argument checks, cached per-(device,
// stream) workspaces, kernel dispatch and error reporting.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stdlib.h>

#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/ssmscan.h"
#include "internal.h"
#include "s6_internal.h"

namespace ssm {

namespace {
thread_local std::string g_last_error;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The byte ranges [p, p + pb) and [q, q + qb) share memory (q may be null).
bool overlap(const void *p, size_t pb, const void *q, size_t qb) {
  if (!p || !q) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + qb && b < a + pb;
}

// Workspace of the look-back linear scan for one (device, stream): the
// claims word, the wave count of a cycle's last launch and the tile status
// words. Never reset between launches: each launch takes a fresh epoch from
// the claims word on the device (so graph replays do too), and the launch
// that ends an epoch cycle clears the words itself.
struct LinearWorkspace {
  AggWord *words = nullptr;  // counters and the three status levels (see linear_workspace)
  int64_t capacity = 0;      // tiles
  uint32_t epoch_cycle = 0;  // fixed when the words are created
};

static_assert(LinearStatus::kDoneOffset * sizeof(unsigned long long) == 128,
              "the done count sits 128 bytes into the 256-byte counter header");
// Epochs are 31-bit (bit 31 of a status word's high half is the batched
// scan's head flag). SSMSCAN_LINEAR_EPOCH_CYCLE, read when a workspace is
// created, shortens the cycle so that tests can exercise the clearing.
constexpr uint32_t kDefaultEpochCycle = 0x7fffffffu;

uint32_t epoch_cycle_for_new_workspace() {
  if (const char *env = getenv("SSMSCAN_LINEAR_EPOCH_CYCLE")) {
    const long long v = atoll(env);
    if (v >= 1 && v <= (long long)kDefaultEpochCycle) return uint32_t(v);
  }
  return kDefaultEpochCycle;
}

struct S6Workspace {
  void *buf = nullptr;
  size_t bytes = 0;
};

// Plain scratch memory for one (device, stream), grown on demand.
struct ScratchWorkspace {
  void *buf = nullptr;
  size_t bytes = 0;
};

using Key = std::pair<int, hipStream_t>;
std::mutex g_mu;
// Buffers replaced by a larger one, per device. A call recorded in a HIP graph
// keeps the buffer it was recorded with, so a replaced buffer stays allocated
// until ssm_release_workspace (growth is geometric: at most as much again as
// the buffers in use).
std::vector<std::pair<int, void *>> g_retired;
std::map<Key, LinearWorkspace> g_linear;
std::map<Key, S6Workspace> g_s6;
std::map<Key, ScratchWorkspace> g_scratch;
std::map<int, int> g_linear_grid;  // device -> resident workgroups of the scan kernel

int current_device(int *dev) {
  return hip_check(hipGetDevice(dev), "hipGetDevice");
}
}  // namespace

int fail(int code, const std::string &msg) {
  g_last_error = msg;
  return code;
}

int hip_check(hipError_t e, const char *what) {
  if (e == hipSuccess) return SSM_OK;
  return fail(SSM_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// A workspace is created or grown only outside HIP graph capture: its
// allocation and zeroing cannot be recorded. Fails when `stream` is capturing.
static int growth_allowed(hipStream_t stream, const char *what) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();  // not sticky; keep it from reaching the next launch check
    return SSM_OK;
  }
  if (cs == hipStreamCaptureStatusNone) return SSM_OK;
  return fail(SSM_ERR_INVALID_ARG,
              std::string(what) + " must be created or grown by a call outside graph capture "
                                  "(make one call of at least this size on the stream first)");
}

// Returns a workspace holding at least `ntiles` status entries, plus the
// number of workgroups to launch.
static int linear_workspace(hipStream_t stream, int64_t ntiles, LinearStatus *status,
                            int *grid) {
  int dev = 0;
  if (int rc = current_device(&dev)) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  auto git = g_linear_grid.find(dev);
  if (git == g_linear_grid.end()) {
    int cus = 0;
    if (int rc = hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                                                 dev), "hipDeviceGetAttribute"))
      return rc;
    int per_cu = linear_wgs_per_cu();
    if (per_cu <= 0) return fail(SSM_ERR_HIP, "occupancy query for the scan kernel failed");
    if (const char *env = getenv("SSMSCAN_LINEAR_WGS_PER_CU")) {
      const int v = atoi(env);
      if (v > 0 && v < per_cu) per_cu = v;
    }
    git = g_linear_grid.emplace(dev, cus * per_cu).first;
  }
  *grid = git->second;
  LinearWorkspace &ws = g_linear[Key(dev, stream)];
  // Layout (each part 256-byte aligned so that the polled status words and
  // the contended counters never share a cache line):
  //   [claims word, done count at +128][level 0: cap][level 1: cap/64]
  //   [level 2: cap/4096] entries.
  auto pad = [](int64_t entries) { return (entries * int64_t(sizeof(AggWord)) + 255) / 256 * 256; };
  auto bytes_for = [&](int64_t cap) { return 256 + pad(cap) + pad(cap / 64) + pad(cap / 4096); };
  if (ws.capacity < ntiles) {
    if (int rc = growth_allowed(stream, "the linear-scan workspace")) return rc;
    if (ws.words) {
      g_retired.emplace_back(dev, ws.words);  // queued or recorded launches may still use it
      ws.words = nullptr;
      ws.capacity = 0;
    }
    int64_t cap = 4096;
    while (cap < ntiles) cap *= 2;
    const size_t bytes = size_t(bytes_for(cap));
    void *p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess)
      return fail(SSM_ERR_ALLOC, "hipMalloc of the linear-scan workspace failed");
    // Zero = epoch 0 everywhere (never written), and the claims word at
    // epoch 1 with nothing claimed.
    if (int rc = hip_check(hipMemsetAsync(p, 0, bytes, stream), "hipMemsetAsync")) {
      (void)hipFree(p);
      return rc;
    }
    ws.words = static_cast<AggWord *>(p);
    ws.capacity = cap;
    ws.epoch_cycle = epoch_cycle_for_new_workspace();
  }
  char *base = reinterpret_cast<char *>(ws.words);
  status->claims = reinterpret_cast<unsigned long long *>(base);  // done count at +128
  status->lvl0 = reinterpret_cast<AggWord *>(base + 256);
  status->lvl1 = reinterpret_cast<AggWord *>(base + 256 + pad(ws.capacity));
  status->lvl2 = reinterpret_cast<AggWord *>(base + 256 + pad(ws.capacity) + pad(ws.capacity / 64));
  status->nwords = (bytes_for(ws.capacity) - 256) / int64_t(sizeof(uint64_t));
  status->epoch_cycle = ws.epoch_cycle;
  return SSM_OK;
}

int s6_workspace(hipStream_t stream, size_t bytes, void **buf) {
  int dev = 0;
  if (int rc = current_device(&dev)) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  S6Workspace &ws = g_s6[Key(dev, stream)];
  if (ws.bytes < bytes || ws.buf == nullptr) {
    if (int rc = growth_allowed(stream, "the S6 workspace")) return rc;
    if (ws.buf) {
      g_retired.emplace_back(dev, ws.buf);  // queued or recorded launches may still use it
      ws.buf = nullptr;
      ws.bytes = 0;
    }
    size_t cap = 1 << 20;
    while (cap < bytes) cap *= 2;
    void *p = nullptr;
    if (hipMalloc(&p, cap) != hipSuccess)
      return fail(SSM_ERR_ALLOC, "hipMalloc of the S6 workspace failed");
    if (int rc = hip_check(hipMemsetAsync(p, 0, cap, stream), "hipMemsetAsync")) {
      (void)hipFree(p);
      return rc;
    }
    ws.buf = p;
    ws.bytes = cap;
  }
  *buf = ws.buf;
  return SSM_OK;
}

// Cached scratch buffer for (current device, stream), at least `bytes` long
// and 256-byte aligned.
static int scratch_workspace(hipStream_t stream, size_t bytes, void **buf) {
  int dev = 0;
  if (int rc = current_device(&dev)) return rc;
  std::lock_guard<std::mutex> lock(g_mu);
  ScratchWorkspace &ws = g_scratch[Key(dev, stream)];
  if (ws.bytes < bytes || ws.buf == nullptr) {
    if (int rc = growth_allowed(stream, "the scratch workspace")) return rc;
    if (ws.buf) {
      g_retired.emplace_back(dev, ws.buf);  // queued or recorded launches may still use it
      ws.buf = nullptr;
      ws.bytes = 0;
    }
    size_t cap = 1 << 20;
    while (cap < bytes) cap *= 2;
    void *p = nullptr;
    if (hipMalloc(&p, cap) != hipSuccess)
      return fail(SSM_ERR_ALLOC, "hipMalloc of the scratch workspace failed");
    ws.buf = p;
    ws.bytes = cap;
  }
  *buf = ws.buf;
  return SSM_OK;
}

}  // namespace ssm

using namespace ssm;

extern "C" {

int ssm_linear_scan(const float *a, const float *b, float h0, float *h, int64_t n,
                    void *stream) {
  g_last_error.clear();
  if (n < 0) return fail(SSM_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return SSM_OK;
  if (!a || !b || !h) return fail(SSM_ERR_INVALID_ARG, "null pointer with n > 0");
  if (!aligned16(a) || !aligned16(b) || !aligned16(h))
    return fail(SSM_ERR_INVALID_ARG, "a, b and h must be 16-byte aligned");
  const int64_t tile = linear_tile_elems(false);
  const int64_t ntiles = (n + tile - 1) / tile;
  if (ntiles > kLinearMaxTiles)
    return fail(SSM_ERR_UNSUPPORTED, "n too large for one launch (max 2^31 elements)");
  const size_t bytes = size_t(n) * sizeof(float);
  if (overlap(h, bytes, a, bytes) || overlap(h, bytes, b, bytes))
    return fail(SSM_ERR_INVALID_ARG, "h overlaps a or b");
  LinearStatus status{};
  int grid = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int rc = linear_workspace(s, ntiles, &status, &grid)) return rc;
  return hip_check(launch_linear_scan(a, b, h0, h, n, ntiles, status, grid, nullptr,
                                      nullptr, 0, s),
                   "linear_scan launch");
}

int ssm_linear_scan_noalloc(const float *a, const float *b, float h0, float *h, int64_t n,
                            void *stream) {
  g_last_error.clear();
  if (n < 0) return fail(SSM_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return SSM_OK;
  if (!a || !b || !h) return fail(SSM_ERR_INVALID_ARG, "null pointer with n > 0");
  if (!aligned16(a) || !aligned16(b) || !aligned16(h))
    return fail(SSM_ERR_INVALID_ARG, "a, b and h must be 16-byte aligned");
  const int64_t tile = linear_tile_elems(false);
  const int64_t ntiles = (n + tile - 1) / tile;
  if (ntiles > kLinearMaxTiles)
    return fail(SSM_ERR_UNSUPPORTED,
                "n too large for the allocation-free scan (its status memory holds 2^31 elements)");
  const size_t bytes = size_t(n) * sizeof(float);
  if (overlap(h, bytes, a, bytes) || overlap(h, bytes, b, bytes))
    return fail(SSM_ERR_INVALID_ARG, "h overlaps a or b");
  // Resident workgroups per device, kept in a fixed table (nothing allocated).
  constexpr int kMaxDevices = 64;
  static int grids[kMaxDevices];
  static std::mutex grid_mu;
  int dev = 0;
  if (int rc = current_device(&dev)) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(SSM_ERR_UNSUPPORTED, "device index too large");
  int grid = 0;
  {
    std::lock_guard<std::mutex> lock(grid_mu);
    if (grids[dev] == 0) {
      int cus = 0;
      if (int rc = hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                                                   dev), "hipDeviceGetAttribute"))
        return rc;
      int per_cu = linear_wgs_per_cu();
      if (per_cu <= 0) return fail(SSM_ERR_HIP, "occupancy query for the scan kernel failed");
      grids[dev] = cus * per_cu;
    }
    grid = grids[dev];
  }
  // The status memory's epochs always use the default cycle: it lives as
  // long as the process, so its cycle cannot change under it.
  LinearStatus status{};
  if (!linear_noalloc_status(&status, kDefaultEpochCycle))
    return fail(SSM_ERR_HIP, "looking up the allocation-free scan's status memory failed");
  return hip_check(launch_linear_scan(a, b, h0, h, n, ntiles, status, grid, nullptr, nullptr, 0,
                                      static_cast<hipStream_t>(stream)),
                   "linear_scan_noalloc launch");
}

int ssm_linear_scan_batched(const float *a, const float *b, const float *h0, float *h,
                            float *h_last, int64_t nseq, int64_t len, void *stream) {
  g_last_error.clear();
  if (nseq < 0 || len < 0) return fail(SSM_ERR_INVALID_ARG, "nseq and len must be >= 0");
  if (nseq == 0 || len == 0) return SSM_OK;
  if (!a || !b || !h) return fail(SSM_ERR_INVALID_ARG, "null a, b or h with work to do");
  if (!aligned16(a) || !aligned16(b) || !aligned16(h))
    return fail(SSM_ERR_INVALID_ARG, "a, b and h must be 16-byte aligned");
  if (nseq > (int64_t(1) << 31) / len)
    return fail(SSM_ERR_UNSUPPORTED, "nseq * len too large for one launch (max 2^31 elements)");
  const int64_t n = nseq * len;
  const size_t bytes = size_t(n) * sizeof(float), sbytes = size_t(nseq) * sizeof(float);
  if (overlap(h, bytes, a, bytes) || overlap(h, bytes, b, bytes) || overlap(h, bytes, h0, sbytes))
    return fail(SSM_ERR_INVALID_ARG, "h overlaps a, b or h0");
  if (overlap(h_last, sbytes, a, bytes) || overlap(h_last, sbytes, b, bytes) ||
      overlap(h_last, sbytes, h, bytes) || overlap(h_last, sbytes, h0, sbytes))
    return fail(SSM_ERR_INVALID_ARG, "h_last overlaps a, b, h or h0");
  const int64_t tile = linear_tile_elems(true);
  const int64_t ntiles = (n + tile - 1) / tile;
  LinearStatus status{};
  int grid = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int rc = linear_workspace(s, ntiles, &status, &grid)) return rc;
  return hip_check(launch_linear_scan(a, b, 0.0f, h, n, ntiles, status, grid, h0, h_last,
                                      uint32_t(len), s),
                   "linear_scan_batched launch");
}

static int linear_3pass_common(const float *a, const float *b, float h0, float *h, int64_t n,
                               bool hillis_steele, void *stream) {
  g_last_error.clear();
  if (n < 0) return fail(SSM_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return SSM_OK;
  if (!a || !b || !h) return fail(SSM_ERR_INVALID_ARG, "null pointer with n > 0");
  if (!aligned16(a) || !aligned16(b) || !aligned16(h))
    return fail(SSM_ERR_INVALID_ARG, "a, b and h must be 16-byte aligned");
  if (n > (int64_t(1) << 31)) return fail(SSM_ERR_UNSUPPORTED, "n too large (max 2^31 elements)");
  const size_t bytes = size_t(n) * sizeof(float);
  if (overlap(h, bytes, a, bytes) || overlap(h, bytes, b, bytes))
    return fail(SSM_ERR_INVALID_ARG, "h overlaps a or b");
  hipStream_t s = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  if (int rc = scratch_workspace(s, linear3_workspace_bytes(n), &ws)) return rc;
  return hip_check(launch_linear_scan_3pass(a, b, h0, h, n, ws, hillis_steele, s),
                   "linear_scan_3pass launch");
}

int ssm_linear_scan_3pass(const float *a, const float *b, float h0, float *h, int64_t n,
                          void *stream) {
  return linear_3pass_common(a, b, h0, h, n, false, stream);
}

int ssm_linear_scan_hs(const float *a, const float *b, float h0, float *h, int64_t n,
                       void *stream) {
  return linear_3pass_common(a, b, h0, h, n, true, stream);
}

int ssm_copy_f32(const float *src, float *dst, int64_t n, void *stream) {
  g_last_error.clear();
  if (n < 0) return fail(SSM_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return SSM_OK;
  if (!src || !dst) return fail(SSM_ERR_INVALID_ARG, "null pointer with n > 0");
  if (!aligned16(src) || !aligned16(dst))
    return fail(SSM_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
  if (overlap(dst, size_t(n) * sizeof(float), src, size_t(n) * sizeof(float)))
    return fail(SSM_ERR_INVALID_ARG, "dst overlaps src");
  return hip_check(launch_copy_f32(src, dst, n, static_cast<hipStream_t>(stream)),
                   "copy launch");
}

int ssm_stream_mul_f32(const float *a, const float *b, float *h, int64_t n, void *stream) {
  g_last_error.clear();
  if (n < 0) return fail(SSM_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return SSM_OK;
  if (n > (int64_t(1) << 40)) return fail(SSM_ERR_UNSUPPORTED, "n above 2^40");
  if (!a || !b || !h) return fail(SSM_ERR_INVALID_ARG, "null pointer with n > 0");
  if (!aligned16(a) || !aligned16(b) || !aligned16(h))
    return fail(SSM_ERR_INVALID_ARG, "a, b and h must be 16-byte aligned");
  const size_t bytes = size_t(n) * sizeof(float);
  if (overlap(h, bytes, a, bytes) || overlap(h, bytes, b, bytes))
    return fail(SSM_ERR_INVALID_ARG, "h overlaps a or b");
  return hip_check(launch_stream_mul_f32(a, b, h, n, static_cast<hipStream_t>(stream)),
                   "stream launch");
}

static int s6_check(const void *u, const void *delta, const float *A, const void *B,
                    const void *C, const float *D, float *y, int batch, int L, int d_inner,
                    int N, int direction, size_t esize, bool *noop) {
  *noop = false;
  if (batch < 0 || L < 0 || d_inner < 0 || N < 0)
    return fail(SSM_ERR_INVALID_ARG, "sizes must be >= 0");
  if (direction < SSM_DIR_FWD || direction > SSM_DIR_BIDIR)
    return fail(SSM_ERR_INVALID_ARG, "direction must be 0 (fwd), 1 (rev) or 2 (bidir)");
  if (N == 0) return fail(SSM_ERR_UNSUPPORTED, "N must be in 1..16");
  if (N > kS6MaxN) return fail(SSM_ERR_UNSUPPORTED, "N must be in 1..16");
  if (batch == 0 || L == 0 || d_inner == 0) {
    *noop = true;
    return SSM_OK;
  }
  if (!u || !delta || !A || !B || !C || !D || !y)
    return fail(SSM_ERR_INVALID_ARG, "null pointer with non-zero sizes");
  const void *ptrs[] = {u, delta, A, B, C, D, y};
  for (const void *p : ptrs)
    if (!aligned16(p)) return fail(SSM_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (int64_t(batch) * L * d_inner > (int64_t(1) << 40))
    return fail(SSM_ERR_UNSUPPORTED, "problem too large");
  const size_t e = size_t(batch) * size_t(L) * size_t(d_inner);  // (b, t, d) elements
  const size_t r = size_t(batch) * size_t(L) * size_t(N);        // (b, t, n) elements
  const size_t yb = e * sizeof(float);
  if (overlap(y, yb, u, e * esize) || overlap(y, yb, delta, e * esize) ||
      overlap(y, yb, B, r * esize) || overlap(y, yb, C, r * esize) ||
      overlap(y, yb, A, size_t(d_inner) * N * sizeof(float)) ||
      overlap(y, yb, D, size_t(d_inner) * sizeof(float)))
    return fail(SSM_ERR_INVALID_ARG, "y overlaps an input");
  return SSM_OK;
}

int ssm_selective_scan_fwd(const float *u, const float *delta, const float *A,
                           const float *B, const float *C, const float *D, float *y,
                           int batch, int L, int d_inner, int N, int direction,
                           void *stream) {
  g_last_error.clear();
  bool noop = false;
  if (int rc = s6_check(u, delta, A, B, C, D, y, batch, L, d_inner, N, direction, 4, &noop))
    return rc;
  if (noop) return SSM_OK;
  S6Args args{u, delta, A, B, C, D, y, batch, L, d_inner, N, direction, false, false, nullptr};
  return run_s6(args, static_cast<hipStream_t>(stream));
}

int ssm_selective_scan_fwd_bf16(const uint16_t *u, const uint16_t *delta, const float *A,
                                const uint16_t *B, const uint16_t *C, const float *D,
                                float *y, int batch, int L, int d_inner, int N,
                                int direction, void *stream) {
  g_last_error.clear();
  bool noop = false;
  if (int rc = s6_check(u, delta, A, B, C, D, y, batch, L, d_inner, N, direction, 2, &noop))
    return rc;
  if (noop) return SSM_OK;
  S6Args args{u, delta, A, B, C, D, y, batch, L, d_inner, N, direction, true, false, nullptr};
  return run_s6(args, static_cast<hipStream_t>(stream));
}

int ssm_selective_scan_fwd_ex(const void *u, const void *delta, const float *delta_bias,
                              const float *A, const void *B, const void *C, const float *D,
                              float *y, int batch, int L, int d_inner, int N, int direction,
                              unsigned flags, void *stream) {
  g_last_error.clear();
  if (flags & ~unsigned(SSM_FLAG_BF16 | SSM_FLAG_DELTA_SOFTPLUS))
    return fail(SSM_ERR_INVALID_ARG, "unknown flag bits");
  const bool softplus = (flags & SSM_FLAG_DELTA_SOFTPLUS) != 0;
  if (delta_bias && !softplus)
    return fail(SSM_ERR_INVALID_ARG, "delta_bias is only applied with SSM_FLAG_DELTA_SOFTPLUS");
  bool noop = false;
  const size_t esize = (flags & SSM_FLAG_BF16) ? 2 : 4;
  if (int rc = s6_check(u, delta, A, B, C, D, y, batch, L, d_inner, N, direction, esize, &noop))
    return rc;
  if (noop) return SSM_OK;
  if (delta_bias && !aligned16(delta_bias))
    return fail(SSM_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
  if (overlap(y, size_t(batch) * size_t(L) * size_t(d_inner) * sizeof(float), delta_bias,
              size_t(d_inner) * sizeof(float)))
    return fail(SSM_ERR_INVALID_ARG, "y overlaps an input");
  S6Args args{u,     delta,    A, B, C, D, y, batch, L, d_inner, N, direction,
              (flags & SSM_FLAG_BF16) != 0, softplus, delta_bias};
  return run_s6(args, static_cast<hipStream_t>(stream));
}

const char *ssm_status_string(int code) {
  switch (code) {
    case SSM_OK: return "ok";
    case SSM_ERR_INVALID_ARG: return "invalid argument";
    case SSM_ERR_UNSUPPORTED: return "unsupported argument";
    case SSM_ERR_HIP: return "HIP runtime error";
    case SSM_ERR_ALLOC: return "workspace allocation failed";
    default: return "unknown status code";
  }
}

const char *ssm_last_error(void) { return g_last_error.c_str(); }

int ssm_release_workspace(void) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lock(g_mu);
  int rc = SSM_OK;
  int saved = 0;
  (void)hipGetDevice(&saved);
  // Wait for every device that owns a workspace (not for its streams: a
  // stream the caller has destroyed since would be an invalid handle).
  std::map<int, bool> devices;
  for (auto &kv : g_linear) devices[kv.first.first] = true;
  for (auto &kv : g_s6) devices[kv.first.first] = true;
  for (auto &kv : g_scratch) devices[kv.first.first] = true;
  for (auto &r : g_retired) devices[r.first] = true;
  for (auto &dv : devices) {
    if (hipSetDevice(dv.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
      rc = fail(SSM_ERR_HIP, "hipDeviceSynchronize failed while releasing workspaces");
  }
  for (auto &kv : g_linear) {
    if (!kv.second.words) continue;
    (void)hipSetDevice(kv.first.first);
    (void)hipFree(kv.second.words);
  }
  for (auto &kv : g_s6) {
    if (!kv.second.buf) continue;
    (void)hipSetDevice(kv.first.first);
    (void)hipFree(kv.second.buf);
  }
  for (auto &kv : g_scratch) {
    if (!kv.second.buf) continue;
    (void)hipSetDevice(kv.first.first);
    (void)hipFree(kv.second.buf);
  }
  for (auto &r : g_retired) {
    (void)hipSetDevice(r.first);
    (void)hipFree(r.second);
  }
  g_linear.clear();
  g_s6.clear();
  g_scratch.clear();
  g_retired.clear();
  (void)hipSetDevice(saved);
  return rc;
}

}  // extern "C"
