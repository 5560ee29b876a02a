/*
 * libssmscan — affine linear-recurrence scan and S6 selective scan for
 * AMD Instinct MI355X (gfx950).
 *
 * C ABI. Every pointer argument is a DEVICE pointer owned by the caller; the
 * library never frees or retains it past the call. Work is enqueued on
 * `stream` (a hipStream_t passed as void*; NULL means the default stream) and
 * the call returns without synchronising. Outputs are fully overwritten and
 * must not overlap any input or each other (checked from the pointers and
 * sizes: SSM_ERR_INVALID_ARG). Every pointer to data must be 16-byte aligned.
 *
 * Return codes (ssm_status_t): SSM_OK on success; on any error nothing is
 * launched and ssm_last_error() describes the cause (per calling thread).
 *
 * Environment (for experiments and verification):
 *   SSMSCAN_S6_CHUNK=<steps>       S6 chunk length, read at every call (kept
 *                                  to at most 256 chunks per sequence; the
 *                                  rounding then follows the new chunks).
 *   SSMSCAN_S6_FULL_FIX=1          S6 evaluates every carry term, read at
 *                                  every call. By default the fix pass leaves
 *                                  out the tail of the decaying carry terms
 *                                  once a bound proves each left-out group of
 *                                  4 states below 2^-24 over a block of
 *                                  steps: outputs differ from full evaluation
 *                                  by at most 2^-22 per direction.
 *   SSMSCAN_LINEAR_WGS_PER_CU=<k>  caps the workgroups per CU of the single-
 *                                  pass linear scan (read once per device).
 *   SSMSCAN_LINEAR_EPOCH_CYCLE=<c> epochs per cycle of the single-pass scans'
 *                                  status words (1 .. 2^31 - 1, the default),
 *                                  read when a stream's workspace is created;
 *                                  a short cycle exercises the launch that
 *                                  clears the words. Results do not depend
 *                                  on it.
 */
#ifndef SSMSCAN_H
#define SSMSCAN_H

#include <stdint.h>

/* The library is built with hidden visibility: only these entry points are
 * exported, so two builds loaded into one process never bind each other's
 * internal functions. */
#define SSM_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative size, bad enum */
  SSM_ERR_UNSUPPORTED = -2, /* valid but not supported here (e.g. N too large) */
  SSM_ERR_HIP = -3,         /* a HIP runtime call failed; see ssm_last_error() */
  SSM_ERR_ALLOC = -4        /* workspace allocation failed */
} ssm_status_t;

typedef enum {
  SSM_DIR_FWD = 0,   /* h[t] from h[t-1], t = 0 .. L-1 */
  SSM_DIR_REV = 1,   /* h[t] from h[t+1], t = L-1 .. 0 */
  SSM_DIR_BIDIR = 2  /* y = y_fwd + y_rev, both directions in one call */
} ssm_direction_t;

/*
 * First-order linear recurrence, as an inclusive prefix scan over affine maps.
 *
 * Defined by "Selective-scan CUDA kernels" (persus.netlify.app/projects/
 * selective-scan), the paragraph stating h[t] = a[t]*h[t-1] + b[t] and its
 * reading as a prefix scan over affine pairs (associative, not commutative).
 *
 *   h[-1] = h0;  h[t] = a[t] * h[t-1] + b[t]   for t = 0 .. n-1
 *
 * a, b : const float[n], input coefficients (fp32, contiguous).
 * h0   : carry-in value.
 * h    : float[n], output (every h[t]); must not overlap a or b.
 * n    : number of elements, n >= 0; n == 0 is a no-op returning SSM_OK.
 *
 * Single pass: each element is read once and written once. The result is
 * bitwise identical from run to run (the cross-tile carry is always folded in
 * the same left-to-right order). It is not bitwise equal to a sequential fp32
 * loop: partial products are associated differently.
 * Non-finite inputs (and h0) give the values the sequential loop gives, inf
 * and NaN in the same places: a product of multipliers that underflows in
 * fp32 is kept as the smallest subnormal of its sign, never 0, so an infinite
 * state pushed through it stays infinite, while an exactly-zero multiplier
 * acts as in the loop (0 times an infinite state is NaN). Products of
 * multipliers above 1 that overflow are outside this guarantee.
 * Uses a library-owned workspace cached per (device, stream): counters and
 * epoch-tagged status words that every launch leaves ready for the next, the
 * epoch advancing on the device. So once a call on `stream` has sized that
 * stream's workspace, a call of the same or smaller size only enqueues one
 * kernel and may be recorded in a HIP graph and replayed (the same holds for
 * ssm_linear_scan_batched). Launches on one workspace must not overlap: calls
 * on one stream are ordered by it, and replays of a recorded call must be
 * ordered with each other and with calls on the stream it was recorded on
 * (overlapping launches can corrupt the counters and leave a later launch
 * waiting forever). A call that would create or grow the workspace during
 * capture fails with SSM_ERR_INVALID_ARG. A larger call moves the stream to
 * a new workspace and keeps the old one, which recorded calls go on using,
 * until ssm_release_workspace: a graph must not be replayed after that.
 * Errors: SSM_ERR_INVALID_ARG for n < 0, null or non-16-byte-aligned a, b, h
 * with n > 0, or h overlapping a or b; SSM_ERR_ALLOC / SSM_ERR_HIP on
 * runtime failure.
 */
SSM_API int ssm_linear_scan(const float *a, const float *b, float h0, float *h, int64_t n,
                            void *stream);

/*
 * ssm_linear_scan for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same recurrence, arguments, result bits and errors as ssm_linear_scan, but
 * the look-back status words live in a fixed device array inside the
 * library (about 4.3 MB per GPU, held until the process ends; its address is
 * looked up once per device), so a call allocates nothing, frees nothing and
 * sets no memory: it only enqueues the scan kernel. The array holds every
 * size ssm_linear_scan accepts (n <= 2^31; larger n returns
 * SSM_ERR_UNSUPPORTED). Every call on a GPU shares that GPU's array, on any
 * stream: calls whose kernels overlap in time on one GPU race and can leave
 * a later call waiting forever, so order them (one stream, or events).
 */
SSM_API int ssm_linear_scan_noalloc(const float *a, const float *b, float h0, float *h,
                                    int64_t n, void *stream);

/*
 * Batched form: nseq independent sequences of `len` elements each, stored one
 * after another (a, b, h are float[nseq][len]), for per-sequence carry-in and
 * carry-out -- e.g. the cross-chunk carries of a chunked scan, or a long
 * sequence resumed in pieces ("Selective-scan CUDA kernels", the recurrence
 * paragraph; the chunked carry scan of "ARM-Scan — Optimized Mamba
 * Selective-Scan Kernel", "Approach"):
 *
 *   h[k][-1] = h0[k];  h[k][t] = a[k][t] * h[k][t-1] + b[k][t]
 *
 * h0     : const float[nseq] or NULL (all sequences start from 0).
 * h_last : float[nseq] or NULL; receives h[k][len-1].
 * One single-pass launch whatever the shape (the sequences are segments of one
 * look-back scan). Deterministic. Every sequence starts from its own h0
 * whatever the previous one ended with (inf and NaN included): sequence
 * starts are marked explicitly, not inferred from zero multipliers. Inside a
 * sequence values, non-finite ones included, are as ssm_linear_scan gives.
 * Errors: SSM_ERR_INVALID_ARG for negative sizes, a null / misaligned a, b,
 * h with work to do, or h / h_last overlapping an input or each other;
 * SSM_ERR_UNSUPPORTED for nseq * len > 2^31; nseq == 0 or len == 0 is a
 * no-op.
 */
SSM_API int ssm_linear_scan_batched(const float *a, const float *b, const float *h0, float *h,
                                    float *h_last, int64_t nseq, int64_t len, void *stream);

/*
 * The same recurrence and arguments as ssm_linear_scan, computed by the
 * three-pass multi-block design that "Selective-scan CUDA kernels" measures
 * its single-pass look-back against (the introduction's memory-traffic model:
 * a 2.33x predicted gain, 2.18-2.48x measured): a local pass writes every
 * element's in-tile composition (A, B), a carry pass folds the tile
 * aggregates, an apply pass writes h = A * h_in + B. 28 bytes of HBM traffic
 * per element instead of 12. Deterministic; not bitwise equal to
 * ssm_linear_scan (different association). Uses a library-owned scratch
 * workspace of about 8 bytes per element, cached per (device, stream); one
 * replaced by a larger call stays allocated until ssm_release_workspace, so
 * growth can hold up to twice the largest size.
 * Errors: as ssm_linear_scan, and SSM_ERR_UNSUPPORTED for n > 2^31.
 */
SSM_API int ssm_linear_scan_3pass(const float *a, const float *b, float h0, float *h, int64_t n,
                                  void *stream);

/*
 * The same recurrence and arguments, by the three-pass structure above with
 * its local pass done as a register-resident Hillis-Steele scan: every row of
 * 256 elements held in registers is scanned in log2(256) = 8 steps in which
 * each element composes with the one d places back (d = 1, 2, ..., 128), with
 * neighbouring lanes' values exchanged through cross-lane shuffles. This is
 * the kernel form of the Hillis-Steele scan that "Selective-scan CUDA kernels"
 * measured only in PyTorch (its introduction: the comparison "is not a fair
 * one yet"). Same traffic as ssm_linear_scan_3pass; deterministic.
 * Errors: as ssm_linear_scan_3pass.
 */
SSM_API int ssm_linear_scan_hs(const float *a, const float *b, float h0, float *h, int64_t n,
                               void *stream);

/*
 * S6 selective scan, forward / reverse / bidirectional, fp32 inputs.
 *
 * Defined by the POPCORNBENCH transcript FW-GLM-5-1 (level 2, problem 30),
 * problem-statement forward pass: per (b, t, d, n)
 *   dA = exp(delta[b,t,d] * A[d,n]),  dBu = delta[b,t,d] * B[b,t,n] * u[b,t,d],
 *   h[b,d,n] = dA * h[b,d,n] + dBu        (state starts at 0),
 *   y[b,t,d] = sum_n C[b,t,n] * h[b,d,n] + D[d] * u[b,t,d].
 * The reverse direction runs t from L-1 down to 0 with the same dA, dBu; the
 * bidirectional form ("ARM-Scan — Optimized Mamba Selective-Scan Kernel",
 * "Approach") computes both directions in one call from the same inputs and
 * writes y = y_fwd + y_rev (each including its D*u term); each direction's
 * sweep evaluates dA and dBu itself.
 *
 * u, delta : const float[batch][L][d_inner]  (delta is already positive,
 *            i.e. after softplus; it is used as given).
 * A        : const float[d_inner][N].
 * B, C     : const float[batch][L][N].
 * D        : const float[d_inner].
 * y        : float[batch][L][d_inner], output (fp32).
 * direction: ssm_direction_t.
 * The (batch, L, d_inner, N) tensors dA, dBu and h never touch memory.
 * Non-finite inputs give the inf and NaN positions (and signs) of the
 * float64 recurrence: an exponential that flushes to zero in fp32 is kept as
 * the smallest subnormal wherever it may meet an infinite state, and a chunk
 * whose C holds an inf or NaN is evaluated again from its exact incoming
 * states (C infinite makes sum_n C*(local + carry term) differ from the sum
 * of the two parts).
 * Accuracy: with the sequence split into chunks, the carry into a chunk is
 * added as its exact decaying contribution, whose tail is left out once
 * proven below 2^-24 per group of 4 states over a block of steps: outputs
 * are within 2^-22 per direction of evaluating every term, on top of fp32
 * rounding (see SSMSCAN_S6_FULL_FIX).
 * Once a call on `stream` has sized that stream's workspace, a call with the
 * same or smaller sizes only enqueues kernels (no allocation, no memset), so
 * it may be recorded in a HIP graph and replayed (also for the _bf16 and _ex
 * forms); replays and calls on that stream must not overlap (they share the
 * workspace). A call that would create or grow the workspace during capture
 * fails with SSM_ERR_INVALID_ARG; a grown-out workspace stays allocated for
 * the calls recorded with it until ssm_release_workspace, after which their
 * graphs must not be replayed.
 * Errors: SSM_ERR_INVALID_ARG for negative sizes, a bad direction, a
 * null / misaligned pointer with non-zero work, or y overlapping an input;
 * SSM_ERR_UNSUPPORTED for N outside 1..16; zero batch, L or d_inner is a
 * no-op returning SSM_OK (checked after the direction and N).
 */
SSM_API int ssm_selective_scan_fwd(const float *u, const float *delta, const float *A,
                                   const float *B, const float *C, const float *D, float *y,
                                   int batch, int L, int d_inner, int N, int direction,
                                   void *stream);

/*
 * As ssm_selective_scan_fwd, with u, delta, B and C stored as bfloat16 (raw
 * uint16 bit patterns); A, D and y stay fp32 and the state is fp32.
 */
SSM_API int ssm_selective_scan_fwd_bf16(const uint16_t *u, const uint16_t *delta,
                                        const float *A, const uint16_t *B, const uint16_t *C,
                                        const float *D, float *y, int batch, int L,
                                        int d_inner, int N, int direction, void *stream);

/* Flags of ssm_selective_scan_fwd_ex. */
enum {
  SSM_FLAG_BF16 = 1,           /* u, delta, B, C are bfloat16 (raw uint16 bits) */
  SSM_FLAG_DELTA_SOFTPLUS = 2  /* delta <- softplus(delta + delta_bias[d]) as read */
};

/*
 * S6 selective scan with the input activation of delta fused in. The
 * POPCORNBENCH transcript FW-GLM-5-1 (level 2, problem 30) computes
 * delta = softplus(proj_delta(x)) (the projection carrying a bias) before the
 * scan; with SSM_FLAG_DELTA_SOFTPLUS the scan takes the pre-activation values
 * and applies  delta_eff[b,t,d] = log(1 + exp(delta[b,t,d] + delta_bias[d]))
 * itself as it reads them, so the activated delta never goes through memory.
 * Everything else is as ssm_selective_scan_fwd (fp32 inputs) or
 * ssm_selective_scan_fwd_bf16 (SSM_FLAG_BF16).
 *
 * delta_bias : const float[d_inner] or NULL (no bias); only with
 *              SSM_FLAG_DELTA_SOFTPLUS.
 * flags      : OR of SSM_FLAG_*.
 * softplus is evaluated in fp32 as max(x, 0) + log(1 + exp(-|x|)), with a
 * short series where exp(-|x|) < 2^-6.
 * Errors: as ssm_selective_scan_fwd; SSM_ERR_INVALID_ARG also for unknown
 * flag bits and for delta_bias without SSM_FLAG_DELTA_SOFTPLUS.
 */
SSM_API int ssm_selective_scan_fwd_ex(const void *u, const void *delta, const float *delta_bias,
                                      const float *A, const void *B, const void *C, const float *D,
                                      float *y, int batch, int L, int d_inner, int N, int direction,
                                      unsigned flags, void *stream);

/*
 * Device copy dst[i] = src[i], i < n (fp32). A known-simple streaming kernel
 * used by measurement code as the bandwidth reference and as the sentinel
 * that must reproduce its input exactly before a timing sweep counts.
 * Errors: as ssm_linear_scan (dst overlapping src is an invalid argument).
 */
SSM_API int ssm_copy_f32(const float *src, float *dst, int64_t n, void *stream);

/*
 * Device product h[i] = a[i] * b[i], i < n (fp32, IEEE products). The
 * linear scan's HBM traffic -- two streams of n floats read, one written,
 * 12 bytes per element -- without the recurrence, in the launch shape that
 * measured fastest for that traffic on gfx950 (one 16-byte vector per lane,
 * 256 lanes per workgroup, one workgroup per 4 KiB of each stream).
 * Measurement code uses it as the attainable-bandwidth reference for the
 * single-pass scan ("Selective-scan CUDA kernels" compares its scan with
 * the memory system's rate in the same way).
 * Errors: SSM_ERR_INVALID_ARG for n < 0, a null / misaligned pointer with
 * n > 0, or h overlapping a or b; SSM_ERR_UNSUPPORTED for n > 2^40.
 */
SSM_API int ssm_stream_mul_f32(const float *a, const float *b, float *h, int64_t n,
                               void *stream);

/* Static English text for a status code. */
SSM_API const char *ssm_status_string(int code);

/* Detail of the last error raised on the calling thread ("" if none). */
SSM_API const char *ssm_last_error(void);

/* Frees every cached workspace, and those replaced by larger ones, after
 * synchronising the device(s) that own them. Safe to call at any time from a
 * thread with no call in flight; graphs recorded before must not be replayed
 * afterwards. */
SSM_API int ssm_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* SSMSCAN_H */
