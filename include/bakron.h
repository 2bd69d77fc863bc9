/*
 * bakron.h -- C ABI of libbakron.so: two-sided (Kronecker-factored) GPTQ
 * rounding on one AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2608.06291, "BaKron: Efficient Quantization with
 * Kronecker-Factored Hessians", also published as "FastKron"; described on
 * the pith.science review page and the mlsanity.com index page):
 *   A weight matrix W (m x n; rows = outputs, columns = inputs) is rounded
 *   under the quadratic loss ||vec(W) - vec(V)||^2_H with H = A (x) B, where A
 *   (n x n) is the input-side and B (m x m) the output-side factor (review
 *   page, "Assumptions").  With LA, LB the lower Cholesky factors of A^-1 and
 *   B^-1 ("What carries the argument"), rounding entry (i,j) with current
 *   value P produces e = (P - Q(P)) / (LB[i][i] LA[j][j]) and the update
 *   W -= e LB[:,i] LA[:,j]^T (Proposition 3.1), which touches only rows >= i
 *   and columns >= j.  Entries on one anti-diagonal i + j = k are
 *   independent, and a recursion over anti-diagonal ranges batches the
 *   postponed updates into two matrix products (Algorithm 6; "Core claim",
 *   Theorem 3.2; O(m+n) sequential steps, O(mn(m+n)) work).
 *
 * Conventions for every call:
 *   - All matrices are dense, row-major, contiguous, 32-bit float unless noted,
 *     and live in device memory of the current HIP device.  They are owned by
 *     the caller; the library never keeps a pointer after the call returns.
 *   - Inputs are never written.  Outputs must not overlap inputs or each other.
 *   - `ws` is caller-owned device scratch of at least *_workspace_size() bytes,
 *     256-byte aligned.  Its contents on entry do not matter.
 *   - Every call enqueues work on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns without waiting, unless a flag below asks for
 *     timing.  Overlapping calls that share a workspace race.
 *   - The return value reports argument and launch errors (BAKRON_ERR_*), and
 *     bakron_last_error() gives a message for the calling thread.  Errors
 *     found by the kernels are OR-ed as BAKRON_DEV_* bits into the optional
 *     device word `dev_status` (caller zeroes it; read it after synchronising).
 */
#ifndef BAKRON_H
#define BAKRON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define BAKRON_OK 0
#define BAKRON_ERR_INVALID_ARG 1
#define BAKRON_ERR_WORKSPACE 2
#define BAKRON_ERR_HIP 5
#define BAKRON_ERR_UNSUPPORTED_DEVICE 6

/* bits OR-ed into *dev_status by the kernels */
#define BAKRON_DEV_NONFINITE 1  /* a non-finite weight or error term was met */
#define BAKRON_DEV_NOT_PD 2     /* a non-positive pivot in bakron_factor */
#define BAKRON_DEV_SPIN_LIMIT 4 /* a bounded wait inside a kernel gave up (results invalid) */

/* base quantizer kinds (the solver is modular in the base quantizer; review
 * page abstract).  Per-row (output channel) parameters from the ORIGINAL W:
 *   SYM  b in {2,3,4,8}: s_i = max_j |W_ij| / (2^(b-1) - 1), z_i = 0,
 *        codes in [-2^(b-1), 2^(b-1) - 1]
 *   ASYM b in {2,3,4}:   s_i = (max_j W_ij - min_j W_ij) / (2^b - 1),
 *        z_i = clamp(rint(-min_j W_ij / s_i), 0, 2^b - 1), codes in [0, 2^b - 1]
 *   UNIT (bits ignored): s_i = 1, z_i = 0, codes in [-128, 127] (unit grid)
 * s_i = 0 is replaced by 1.  The scale is IEEE fp32 arithmetic on fp32 data.
 * An entry with value P gets code c = clamp(rint(P / s_i) + z_i) (round half
 * to even) and dequantised value v = s_i (c - z_i). */
#define BAKRON_Q_SYM 0
#define BAKRON_Q_ASYM 1
#define BAKRON_Q_UNIT 2

/* flags for bakron_quantize */
#define BAKRON_ORDER_AUTO 0        /* pick the product order with fewer executed flops */
#define BAKRON_ORDER_LA_FIRST 1    /* band update as LB (E_S LA^T) */
#define BAKRON_ORDER_LB_FIRST 2    /* band update as (LB E_S) LA^T */
#define BAKRON_ORDER_MASK 3
#define BAKRON_FLAG_PHASE_TIMING 4 /* time each phase with HIP events; the call
                                      then synchronises the stream before it
                                      returns.  See bakron_last_phase_ms(). */
#define BAKRON_FLAG_NO_GRAPH 8     /* launch kernel by kernel instead of replaying
                                      the cached executable graph of the solve */
#define BAKRON_FLAG_MSE_SCALE 16   /* per-row scale shrink by MSE search (review
                                      page, free parameters: up to a factor 2).
                                      The row's range is scaled by p = 1, 0.99,
                                      ..., 0.50; each candidate takes the plain
                                      parameters of the shrunk range; the first p
                                      with the least sum over the row of
                                      (w - v)^2 (v the clamped base-quantizer value
                                      of w, fp32; sum in fp64) wins.  Symmetric and
                                      asymmetric kinds; ignored for BAKRON_Q_UNIT. */
#define BAKRON_FLAG_SPLIT_COLS 32  /* hybrid schedule (review "Circularity Check":
                                      BaKron-recursive's recurrence, Appendix C): solve
                                      the tile columns 0 .. N/2-1, apply their updates to
                                      the rest (W2 -= LB E1 LA21^T), solve the rest;
                                      each half by the recursion over anti-diagonals.
                                      Same result (Theorem 3.2). */
#define BAKRON_FLAG_SPLIT_ROWS 64  /* the same with the tile rows 0 .. M/2-1 first
                                      (W2 -= LB21 E1 LA^T).  At most one split flag;
                                      neither with BAKRON_FLAG_PHASE_TIMING. */

/*
 * bakron_hessian -- Kronecker factor from samples, with damping.
 *   H = X^T X / N + damp_rel * mean(diag(X^T X / N)) * I
 * (input side: X = activation samples, giving A; output side: output-side
 * samples, giving B.  Gram regularisation by a multiple of the mean diagonal:
 * review page, free parameters.)
 *   X  N x d, row-major (one sample per row), device.   H  d x d, full
 *   symmetric, device.  N >= 1, d >= 1, damp_rel >= 0 and finite.
 * Computed with fp32 matrix cores, fp32 accumulation.
 */
size_t bakron_hessian_workspace_size(int64_t N, int64_t d);
int32_t bakron_hessian(const float *X, int64_t N, int64_t d, float damp_rel,
                       float *H, void *ws, size_t ws_bytes, void *stream);

/*
 * bakron_factor -- L = lower Cholesky factor of H^-1 (L L^T = H^-1), the
 * "normalised Cholesky factor" the solver consumes (review page, "What
 * carries the argument": lower-triangular Cholesky factors of A^-1, B^-1).
 *   H  d x d symmetric positive definite (only the lower triangle is read).
 *   L  d x d lower triangular, strictly-upper part written as 0.
 * Computed in fp64 as the reverse-order factorisation H = U U^T (U upper),
 * L = U^-T.  A non-positive pivot sets BAKRON_DEV_NOT_PD in *dev_status (may
 * be NULL) and leaves L undefined.
 */
size_t bakron_factor_workspace_size(int64_t d);
int32_t bakron_factor(const float *H, int64_t d, float *L, int32_t *dev_status,
                      void *ws, size_t ws_bytes, void *stream);

/*
 * bakron_quantize -- the solver (BaKron, Algorithm 6).
 *   W      m x n input weights.
 *   LA     n x n, lower Cholesky factor of A^-1 (only the lower triangle is read).
 *   LB     m x m, lower Cholesky factor of B^-1 (only the lower triangle is read).
 *   qkind, qbits  base quantizer (BAKRON_Q_*).
 *   codes  m x n int8 output codes.
 *   scales m output per-row scales.       zeros  m per-row zero points or NULL.
 *   V      m x n dequantised output (v = s_i (c - z_i)), or NULL.
 *   E      m x n normalised errors e_ij, or NULL.
 *   sum_e2 device double, receives sum e_ij^2 (= the proxy loss when LA, LB
 *          are exact; fixed-order reduction), or NULL.
 *   flags  BAKRON_ORDER_* | BAKRON_FLAG_*.
 * Any m, n >= 1 is accepted; inside, W is handled in 64 x 64 tiles with
 * zero padding.  The result equals the raster-order naive solver up to fp32
 * rounding order (Theorem 3.2).
 * The static schedule of a solve (see bakron_schedule_plan) runs on two
 * streams: `stream` carries the leaves and the band products that feed the
 * next target diagonals; the rest of the wide recursion nodes' products runs
 * on a side stream of the library's, forked and joined with events, while the
 * leaves occupy few CUs.  The results do not depend on the interleaving (the
 * plan orders every pair of steps that share data) and are the same bit for
 * bit with and without BAKRON_FLAG_NO_GRAPH and BAKRON_FLAG_PHASE_TIMING (the
 * latter runs the plan in order on `stream`).
 * The schedule is captured once into an executable HIP graph, cached per
 * (device, sizes, quantizer, order, every pointer argument, ws) -- at most 16
 * graphs, least recently used dropped -- and replayed on `stream`.  The first
 * call with a new key pays the capture.  Calls from several host threads are
 * safe when they use distinct workspaces and outputs: the cache is locked from
 * lookup through launch, and an evicted graph is destroyed only after its
 * last launch has completed.  Calls that share a workspace race on it.
 */
size_t bakron_quantize_workspace_size(int64_t m, int64_t n, int32_t qkind, int32_t qbits);
int32_t bakron_quantize(const float *W, int64_t m, int64_t n, const float *LA,
                        const float *LB, int32_t qkind, int32_t qbits,
                        int8_t *codes, float *scales, float *zeros, float *V,
                        float *E, double *sum_e2, int32_t *dev_status,
                        int32_t flags, void *ws, size_t ws_bytes, void *stream);

/*
 * bakron_quantize_noalloc -- bakron_quantize for callers that cannot allocate
 * device memory: code under HIP stream capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as bakron_quantize, without
 * the workspace; the flags BAKRON_ORDER_*, BAKRON_FLAG_MSE_SCALE and
 * BAKRON_FLAG_SPLIT_* (BAKRON_FLAG_NO_GRAPH is accepted and changes nothing).
 *   - The solve's scratch is a fixed array of BAKRON_NOALLOC_SCRATCH_BYTES in
 *     device memory, inside the library: each GPU it runs on holds one copy
 *     until the process ends.  A shape whose workspace
 *     (bakron_quantize_workspace_size) exceeds it is rejected with
 *     BAKRON_ERR_WORKSPACE before anything is enqueued (2048 x 2048 fits,
 *     4096 x 4096 does not).
 *   - The plan runs in order on `stream` alone: no side stream, no event, no
 *     graph.  The results equal bakron_quantize's bit for bit.
 *   - It calls no hipMalloc, hipFree or other allocating routine.
 *   - Every call on one GPU uses that GPU's array, which keeps the last call's
 *     contents (what must start at zero is cleared by each call).  Calls that
 *     overlap on one GPU (other streams, other host threads) race on it and
 *     give wrong results: serialise them.
 * Returns as bakron_quantize; BAKRON_FLAG_PHASE_TIMING is rejected.
 */
#define BAKRON_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int32_t bakron_quantize_noalloc(const float *W, int64_t m, int64_t n, const float *LA,
                                const float *LB, int32_t qkind, int32_t qbits, int8_t *codes,
                                float *scales, float *zeros, float *V, float *E, double *sum_e2,
                                int32_t *dev_status, int32_t flags, void *stream);

/*
 * bakron_quantize_antidiag -- BaKron-antidiagonal, the pages' comparison
 * variant (review page "If this is right": BaKron runs about 27x faster than
 * it at 4096 x 4096; "Core claim", Theorem 3.2: both give the same output).
 * Every entry anti-diagonal d = i + j is rounded at once, then its rank-|d|
 * update W[i'][j'] -= sum_{(i,j) on d} LB[i'][i] e_ij LA[j'][j] is applied to
 * the rest of the matrix: O(m + n) steps, O(m^2 n^2) work.  Arguments,
 * quantizer and outputs as for bakron_quantize (no sum_e2; no flags); two
 * kernel launches per anti-diagonal on `stream`, no graph.  Its own workspace
 * (bakron_quantize_antidiag_workspace_size).  Returns as bakron_quantize.
 */
size_t bakron_quantize_antidiag_workspace_size(int64_t m, int64_t n, int32_t qkind, int32_t qbits);
int32_t bakron_quantize_antidiag(const float *W, int64_t m, int64_t n, const float *LA,
                                 const float *LB, int32_t qkind, int32_t qbits, int8_t *codes,
                                 float *scales, float *zeros, float *V, float *E,
                                 int32_t *dev_status, void *ws, size_t ws_bytes, void *stream);

/*
 * bakron_schedule_info -- the static schedule for an m x n solve, without
 * touching the GPU.  out[0..14]:
 *   0 tile size b           1 leaf launches (tile anti-diagonals M+N-1)
 *   2 band GEMM launches    3 sequential in-kernel diagonal steps ((M+N-1)(2b-1))
 *   4 order used (1 = LA first, 2 = LB first)
 *   5 algorithmic band flops: two products per recursion node at single
 *     anti-diagonal granularity (the exact staircase count of Algorithm 6)
 *   6 flops the band GEMM launches execute with dense b x b tiles (order of out[4])
 *   7 the paper's count F = m n (m + n)
 *   8 in-tile leaf flops executed (two length-b dot products per entry)
 *   9 recursion depth (levels)
 *  10 useful flops of the band GEMM launches: out[6] without the zero half of
 *     the triangular diagonal factor blocks
 *  11 flops of the two-diagonal nodes: a recursion node over two tile
 *     diagonals has no launch of its own; its update (up to four dense
 *     b x b x b products per tile) runs inside the leaves of its two diagonals
 *  12 leaf launches that pull
 *  13 of the band launches in out[2]: deferred ones (side stream)
 *  14 useful flops of the deferred launches (part of out[10])
 * Returns BAKRON_OK or BAKRON_ERR_INVALID_ARG.
 */
int32_t bakron_schedule_info(int64_t m, int64_t n, int32_t flags, double *out);

/*
 * bakron_schedule_plan -- the ordered steps of an m x n solve, for inspection
 * and tests; touches no GPU.  Writes *count; with ops != NULL (cap >= *count
 * entries of 16 int32, else BAKRON_ERR_INVALID_ARG) entry k is step k:
 *   [0] kind: 0 leaf, 1 band product, 2 record event, 3 wait for event
 *   [1] band: 1 = deferred (side stream); record / wait: 1 = on the side stream
 *   [2] record / wait: event index
 *   leaf:  [3] tile diagonal K, [4] 1 = applies the previous leaf's
 *          two-diagonal update, 2 = computes it for the next leaf
 *   band:  [3] K, [5] L, [6] H of the recursion node (split at K + H), [7] its
 *          T buffer (its recursion depth; the nodes below the deepest level
 *          that defers products share one), [8] product (0 first, 1 second),
 *          [9..10] diagonal range lo, hi (T diagonals for the first product,
 *          W target diagonals for the second), then the launch grid for the
 *          order given in flags: [11] mode, [12] first band offset, [13] offsets,
 *          [14] first row, [15] rows (-1 when the range holds no tile).
 * Unused fields are -1.  Returns BAKRON_OK or BAKRON_ERR_INVALID_ARG.
 */
int32_t bakron_schedule_plan(int64_t m, int64_t n, int32_t flags, int32_t *ops, int64_t cap,
                             int64_t *count);

/* Per-phase times (ms) of the calling thread's last bakron_quantize call made
 * with BAKRON_FLAG_PHASE_TIMING.  That call runs the plan in order on one
 * stream with an event after every step: out[0] quantizer parameters +
 * relayout, out[1] leaf kernels, out[2] band GEMM kernels on the critical
 * stream, out[3] finalise, out[4] leaf launches, out[5] critical band GEMM
 * launches, out[6] deferred band kernels, out[7] deferred band launches.
 * These intervals include each launch's dispatch latency.  The call then
 * replays the critical band launches alone, and then the deferred ones alone,
 * each as a one-off graph whose kernels start back to back, timed by events
 * around the graph launch: out[8] and out[9] (kernel time without dispatch
 * gaps; the replays rewrite the workspace, not the outputs).  Returns
 * BAKRON_ERR_INVALID_ARG if no such call was made. */
int32_t bakron_last_phase_ms(double *out);

const char *bakron_status_string(int32_t status);
const char *bakron_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BAKRON_H */
