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

// Per-tile status, written with single 64-bit relaxed atomic stores at agent
// scope. Each word carries the launch's 32-bit epoch in its high half and a
// 32-bit float payload in its low half, so a word is either "not yet written
// in this launch" (epoch differs) or complete; no fence pairs are needed and a
// NaN payload cannot be mistaken for a flag.
struct TileStatus {
  uint64_t agg_a;  // (epoch << 32) | bits(tile aggregate multiplier)
  uint64_t agg_b;  // (epoch << 32) | bits(tile aggregate offset)
  uint64_t inc;    // (epoch << 32) | bits(h at the end of the tile)
  uint64_t pad;
};

// Elements per tile of the look-back scan.
int64_t linear_tile_elems();

// Enqueues the single-pass scan. status must hold ntiles entries whose
// epochs differ from `epoch`; *ticket must equal ticket_base at launch start.
hipError_t launch_linear_scan(const float *a, const float *b, float h0, float *h,
                              int64_t n, int64_t ntiles, TileStatus *status,
                              unsigned long long *ticket,
                              unsigned long long ticket_base, uint32_t epoch,
                              hipStream_t stream);

hipError_t launch_copy_f32(const float *src, float *dst, int64_t n,
                           hipStream_t stream);

}  // namespace ssm
