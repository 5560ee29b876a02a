// Internal declarations for the S6 selective-scan path of libssmscan.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssm {

constexpr int kS6MaxN = 16;

struct S6Args {
  const void *u;      // (batch, L, d_inner), fp32 or bf16
  const void *delta;  // (batch, L, d_inner), fp32 or bf16
  const float *A;     // (d_inner, N)
  const void *B;      // (batch, L, N), fp32 or bf16
  const void *C;      // (batch, L, N), fp32 or bf16
  const float *D;     // (d_inner)
  float *y;           // (batch, L, d_inner)
  int batch, L, d_inner, N, direction;
  bool bf16;
  bool delta_softplus;       // delta <- softplus(delta + delta_bias[d]) as it is read
  const float *delta_bias;   // (d_inner) or null; only with delta_softplus
};

// Validated arguments in, kernels enqueued on `stream` out.
int run_s6(const S6Args &args, hipStream_t stream);

// Cached S6 workspace for (current device, stream), at least `bytes` long.
// Allocated (and zeroed) only when it grows; otherwise the call touches no
// memory, so S6 calls that fit the workspace enqueue kernels only.
int s6_workspace(hipStream_t stream, size_t bytes, void **buf);

}  // namespace ssm
