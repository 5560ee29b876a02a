/*
 * Plain C float64 twin of the oracle (test infrastructure only).
 *
 * Used where the Python loops of oracle/linear.py and oracle/s6.py are too slow:
 * full-size parity checks and the CPU baseline. Shares no code, header or
 * constant with the GPU library. Built with -O2 -fno-fast-math
 * -ffp-contract=off so that every a*h+b is a rounded multiply followed by a
 * rounded add, exactly as written.
 *
 * Definitions:
 *  - linear recurrence h[t] = a[t]*h[t-1] + b[t], h[-1] = h0: "Selective-scan
 *    CUDA kernels" (persus.netlify.app), the paragraph stating the recurrence.
 *  - S6 forward: POPCORNBENCH transcript FW-GLM-5-1 (level 2, problem 30),
 *    problem-statement forward pass (dA = exp(delta*A), dB = delta*B,
 *    x_db = x*dB, h = dA*h + x_db, y_t = sum_n h*C_t, y + x*D), state starting
 *    at zero as in its sequential kernel.
 *  - reverse and bidirectional: "ARM-Scan — Optimized Mamba Selective-Scan
 *    Kernel", "Approach": the reverse recurrence reuses the discretized terms;
 *    bidir = fwd + rev, each with its own D*u term.
 *
 * Inputs and outputs are double (fp32 and bf16 data widen to double exactly);
 * all arithmetic is double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

void oracle_linear_scan(const double *a, const double *b, double h0, double *h,
                        int64_t n) {
  double state = h0;
  for (int64_t t = 0; t < n; ++t) {
    state = a[t] * state + b[t];
    h[t] = state;
  }
}

/* One channel (batch index bi, channel d) in one direction; adds into y when
 * accumulate != 0, otherwise overwrites. */
static void s6_channel(const double *u, const double *delta, const double *A,
                       const double *B, const double *C, const double *D, double *y,
                       int64_t L, int64_t d_inner, int64_t N, int64_t bi,
                       int64_t d, int reverse, int accumulate, double *h) {
  for (int64_t n = 0; n < N; ++n) h[n] = 0.0;
  for (int64_t s = 0; s < L; ++s) {
    const int64_t t = reverse ? (L - 1 - s) : s;
    const int64_t e = (bi * L + t) * d_inner + d;
    const double dt = delta[e];
    const double x = u[e];
    const double *Bt = B + (bi * L + t) * N;
    const double *Ct = C + (bi * L + t) * N;
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double dA = exp(dt * A[d * N + n]);
      const double dB = dt * Bt[n];
      const double x_db = x * dB;
      h[n] = dA * h[n] + x_db;
      acc += h[n] * Ct[n];
    }
    const double out = acc + x * D[d];
    y[e] = accumulate ? y[e] + out : out;
  }
}

/* direction: 0 forward, 1 reverse, 2 bidirectional (forward + reverse).
 * Channels [ch_begin, ch_end) of the flattened (batch, d_inner) index are
 * computed; y is the full (batch, L, d_inner) array and only those channels
 * are written. nthreads <= 0 means the OpenMP default.
 * Returns the number of threads used, or -1 on a bad argument. */
int oracle_s6(const double *u, const double *delta, const double *A,
              const double *B, const double *C, const double *D, double *y,
              int64_t batch, int64_t L, int64_t d_inner, int64_t N,
              int direction, int64_t ch_begin, int64_t ch_end, int nthreads) {
  if (direction < 0 || direction > 2 || N <= 0 || N > 4096) return -1;
  if (ch_begin < 0 || ch_end > batch * d_inner || ch_begin > ch_end) return -1;
  int used = 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
    double *h = (double *)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = ch_begin; c < ch_end; ++c) {
      const int64_t bi = c / d_inner, d = c % d_inner;
      if (direction == 0 || direction == 2)
        s6_channel(u, delta, A, B, C, D, y, L, d_inner, N, bi, d, 0, 0, h);
      if (direction == 1)
        s6_channel(u, delta, A, B, C, D, y, L, d_inner, N, bi, d, 1, 0, h);
      if (direction == 2)
        s6_channel(u, delta, A, B, C, D, y, L, d_inner, N, bi, d, 1, 1, h);
    }
    free(h);
  }
#else
  (void)nthreads;
  double *h = (double *)malloc(sizeof(double) * (size_t)N);
  for (int64_t c = ch_begin; c < ch_end; ++c) {
    const int64_t bi = c / d_inner, d = c % d_inner;
    if (direction == 0 || direction == 2)
      s6_channel(u, delta, A, B, C, D, y, L, d_inner, N, bi, d, 0, 0, h);
    if (direction == 1)
      s6_channel(u, delta, A, B, C, D, y, L, d_inner, N, bi, d, 1, 0, h);
    if (direction == 2)
      s6_channel(u, delta, A, B, C, D, y, L, d_inner, N, bi, d, 1, 1, h);
  }
  free(h);
#endif
  return used;
}
