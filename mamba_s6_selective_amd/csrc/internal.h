// Internal declarations shared by the host entry points and the kernel
// launchers of libssmscan. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace ssm {

// Records a message for ssm_last_error() on the calling thread and returns code.
int fail(int code, const std::string &msg);
// Wraps a HIP call result: SSM_OK, or SSM_ERR_HIP with the runtime's text.
int hip_check(hipError_t e, const char *what);

// ---- linear recurrence -----------------------------------------------------

// One published affine aggregate: two 64-bit words written with relaxed
// agent-scope atomic stores. Each word carries the launch's 32-bit epoch in its
// high half and an fp32 payload in its low half, so a word is either "not yet
// written in this launch" (epoch differs) or complete; no fence pairs are
// needed and a NaN payload cannot be mistaken for a flag.
struct AggWord {
  uint64_t a;  // (epoch << 32) | bits(multiplier)
  uint64_t b;  // (epoch << 32) | bits(offset)
};

// Status of one launch: aggregates of tiles (level 0), of superblocks of 64
// tiles (level 1) and of blocks of 64 superblocks (level 2).
struct LinearStatus {
  AggWord *lvl0;
  AggWord *lvl1;
  AggWord *lvl2;
  // ((epoch - 1) << 32) | tiles claimed so far by the launch in progress; the
  // launch's last claim stores the next launch's value. The epoch thus lives
  // on the device, and a launch replayed from a recorded graph still gets a
  // fresh one.
  // claims[kDoneOffset] counts the waves that have finished, only in a
  // launch that ends the epoch cycle.
  unsigned long long *claims;
  int64_t nwords;        // 64-bit words from lvl0 through lvl2 (padding included)
  uint32_t epoch_cycle;  // epochs run 1 .. epoch_cycle, then start again at 1
  static constexpr int kDoneOffset = 16;  // 128 bytes: its own cache line
};

// Largest tile count one launch supports (three levels of 64).
constexpr int64_t kLinearMaxTiles = int64_t(64) * 64 * 64;

// Elements per tile of the look-back scan.
int64_t linear_tile_elems(bool segmented);

// Enqueues the single-pass scan on min(ntiles, resident_wgs) persistent
// workgroups (ntiles >= 1). The status levels must hold ntiles,
// ceil(ntiles/64) and ceil(ntiles/4096) entries whose epochs differ from the
// one *claims gives, *claims' count and *done must be 0 and *claims' epoch
// below epoch_cycle: a zeroed workspace is so, and every launch leaves it so
// for the next. Launches on one workspace must not overlap. seg_len > 0 scans
// n / seg_len independent sequences of seg_len elements (sequence k from seg_h0[k], or 0 if seg_h0 is
// null; its last value to seg_h_last[k] if that is not null); h0 is then
// unused. n < 2^32 with segments.
hipError_t launch_linear_scan(const float *a, const float *b, float h0, float *h,
                              int64_t n, int64_t ntiles, LinearStatus status,
                              int resident_wgs, const float *seg_h0, float *seg_h_last,
                              uint32_t seg_len, hipStream_t stream);
// Workgroups of the scan kernel that fit on one CU at once (0 on error).
int linear_wgs_per_cu();

// Status words of the allocation-free linear scan for the current device (a
// file-scope device array of linear_noalloc_bytes() bytes holding up to
// kLinearMaxTiles tiles; its address is looked up once per device). Returns 1
// on success, 0 if the device or symbol lookup failed.
int linear_noalloc_status(LinearStatus *status, uint32_t epoch_cycle);
size_t linear_noalloc_bytes();

hipError_t launch_copy_f32(const float *src, float *dst, int64_t n,
                           hipStream_t stream);
hipError_t launch_stream_mul_f32(const float *a, const float *b, float *h, int64_t n,
                                 hipStream_t stream);

// ---- three-pass linear recurrence ------------------------------------------

int64_t linear3_tile_elems();
// Device workspace the three-pass scan needs for n elements.
size_t linear3_workspace_bytes(int64_t n);
// Enqueues the local, carry and apply passes; `workspace` holds at least
// linear3_workspace_bytes(n) bytes, 256-byte aligned. hillis_steele selects
// the register-resident Hillis-Steele local pass.
hipError_t launch_linear_scan_3pass(const float *a, const float *b, float h0, float *h,
                                    int64_t n, void *workspace, bool hillis_steele,
                                    hipStream_t stream);

}  // namespace ssm
