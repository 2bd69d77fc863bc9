/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU statement of two-sided (Kronecker-factored)
 * GPTQ rounding, used to check the HIP library.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header or constant with the GPU library.
 *
 * Source of the method: the pith.science review of arXiv 2608.06291
 * ("BaKron: Efficient Quantization with Kronecker-Factored Hessians"),
 * sections "What carries the argument" (Proposition 3.1: the vectorised
 * GPTQ step is the outer product L^B_i * delta * (L^A_j)^T in matrix space,
 * touching only rows >= i and columns >= j) and "Core claim" (Theorem 3.2:
 * the naive, anti-diagonal, recursive and BaKron variants give the same
 * output; entries on one anti-diagonal i+j=k are independent).
 *
 * Conventions (readings; see the design notes):
 *   W  m x n row-major (rows = outputs, columns = inputs)
 *   LA n x n lower, LA LA^T = A^{-1} (input side);  LB m x m lower, LB LB^T = B^{-1}
 *   entry (i,j): P = current value, u = P / s_i (code units),
 *                c = clamp(rint(u) + z_i, qmin, qmax), v = s_i (c - z_i),
 *                e = (P - v) / (LB[i][i] LA[j][j]),
 *                W[i'][j'] -= e LB[i'][i] LA[j'][j]   for i' >= i, j' >= j.
 *   rint is round-half-to-even (the C default rounding mode).
 *
 * Tie adoption ("replay"): when a reference code array is given, an entry
 * whose u lies within `window` code units of an interior rounding boundary
 * takes the reference code if it is one of the two codes adjacent to that
 * boundary.  Such entries are counted as ties; any other disagreement is
 * counted as a mismatch and the oracle keeps its own code.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -shared -fPIC oracle.c -lm
 * (no fused multiply-add, so each step is the plain IEEE operation written).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_SYM 0
#define ORC_ASYM 1
#define ORC_UNIT 2

/* ------------------------------------------------------------------ */
/* quantizer parameters, fp32 semantics, from the ORIGINAL weights.    */
/* Per-row (output channel) scale as on the review page's free-        */
/* parameter list ("per-row scaling factor"), without the MSE shrink.  */
/* Each fp32 operation is done in fp64 and rounded once to fp32, which */
/* is the correctly rounded fp32 result for +, -, * and /.             */
/* ------------------------------------------------------------------ */
int orc_qparams(const float *W, int64_t m, int64_t n, int kind, int bits,
                float *scales, float *zeros)
{
    if (m < 0 || n < 0) return 1;
    for (int64_t i = 0; i < m; i++) {
        const float *row = W + i * n;
        float s, z = 0.0f;
        if (kind == ORC_UNIT) {
            s = 1.0f;
        } else if (kind == ORC_SYM) {
            double amax = 0.0;
            for (int64_t j = 0; j < n; j++) {
                double a = fabs((double)row[j]);
                if (a > amax) amax = a;
            }
            double qmax = (double)((1 << (bits - 1)) - 1);
            s = (float)(amax / qmax);
            if (s == 0.0f) s = 1.0f;
        } else if (kind == ORC_ASYM) {
            double lo = INFINITY, hi = -INFINITY;
            for (int64_t j = 0; j < n; j++) {
                double a = (double)row[j];
                if (a < lo) lo = a;
                if (a > hi) hi = a;
            }
            double qmax = (double)((1 << bits) - 1);
            float range = (float)(hi - lo);
            s = (float)((double)range / qmax);
            if (s == 0.0f) {
                s = 1.0f;
                z = 0.0f;
            } else {
                float t = (float)(-lo / (double)s);
                double zz = rint((double)t);
                if (zz < 0.0) zz = 0.0;
                if (zz > qmax) zz = qmax;
                z = (float)zz;
            }
        } else {
            return 2;
        }
        scales[i] = s;
        zeros[i] = z;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* per-row scale shrink chosen by an MSE search (review page, free     */
/* parameters: the per-row scaling factor is shrunk by up to a factor  */
/* of 2, chosen by an MSE search).  Reading: the candidates are the    */
/* grid's range (max|w| for symmetric, [min w, max w] for asymmetric)  */
/* multiplied by p_k = (grid - k) / grid, k = 0 .. maxk (grid 100,     */
/* maxk 50: p from 1 down to 1/2); each candidate's parameters follow  */
/* the plain rule on the shrunk range; its error is the sum over the   */
/* row of (w - v)^2, v the base quantizer's value of w on that grid    */
/* (clamped); the first candidate with the least error wins (ties keep */
/* the larger p).  fp32 semantics for the parameters and for v, fp64   */
/* for the squared errors and their sum (plain order j = 0 .. n-1).    */
/* k = 0 gives orc_qparams' parameters.                                */
/* kbest (m), errs, cand_s and cand_z (m x (maxk+1): every candidate's */
/* error, scale and zero point) may be NULL.                           */
/* ------------------------------------------------------------------ */
static float f32(double x) { return (float)x; }

int orc_qparams_mse(const float *W, int64_t m, int64_t n, int kind, int bits, int grid,
                    int maxk, float *scales, float *zeros, int32_t *kbest, double *errs,
                    float *cand_s, float *cand_z)
{
    if (m < 0 || n < 1 || grid < 1 || maxk < 0 || maxk >= grid) return 1;
    if (kind != ORC_SYM && kind != ORC_ASYM) return 2;
    const double qmin = kind == ORC_SYM ? -(double)(1 << (bits - 1)) : 0.0;
    const double qmax = kind == ORC_SYM ? (double)((1 << (bits - 1)) - 1) : (double)((1 << bits) - 1);
    for (int64_t i = 0; i < m; i++) {
        const float *row = W + i * n;
        float amax = 0.0f, lo = INFINITY, hi = -INFINITY;
        for (int64_t j = 0; j < n; j++) {
            if (fabsf(row[j]) > amax) amax = fabsf(row[j]);
            if (row[j] < lo) lo = row[j];
            if (row[j] > hi) hi = row[j];
        }
        double best = INFINITY;
        for (int k = 0; k <= maxk; k++) {
            const float p = f32((double)(grid - k) / (double)grid);
            float s, z = 0.0f;
            if (kind == ORC_SYM) {
                s = f32((double)f32((double)amax * p) / qmax);
                if (s == 0.0f) s = 1.0f;
            } else {
                const float lo_p = f32((double)lo * p), hi_p = f32((double)hi * p);
                s = f32((double)f32((double)hi_p - lo_p) / qmax);
                if (s == 0.0f) {
                    s = 1.0f;
                } else {
                    double zz = rint((double)f32(-(double)lo_p / s));
                    if (zz < 0.0) zz = 0.0;
                    if (zz > qmax) zz = qmax;
                    z = (float)zz;
                }
            }
            double err = 0.0;
            for (int64_t j = 0; j < n; j++) {
                double c = rint((double)f32((double)row[j] / s)) + z;
                if (c < qmin) c = qmin;
                if (c > qmax) c = qmax;
                const float v = f32((double)s * (c - z));
                const double d = (double)row[j] - (double)v;
                err += d * d;
            }
            if (errs) errs[i * (maxk + 1) + k] = err;
            if (cand_s) cand_s[i * (maxk + 1) + k] = s;
            if (cand_z) cand_z[i * (maxk + 1) + k] = z;
            if (err < best) {
                best = err;
                scales[i] = s;
                zeros[i] = z;
                if (kbest) kbest[i] = k;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* one rounding decision, with optional adoption of a reference code   */
/* ------------------------------------------------------------------ */
typedef struct {
    int kind, qmin, qmax;
    const int8_t *ref;   /* reference codes, m x n row-major, or NULL */
    double window;
    int64_t ties, mismatches;
} qctx;

static void round_entry(qctx *q, int64_t idx, double P, double s, double z,
                        double *u_out, int *c_out, double *v_out)
{
    double u = P / s;
    double c = rint(u) + z;
    if (c < q->qmin) c = q->qmin;
    if (c > q->qmax) c = q->qmax;
    int code = (int)c;
    if (q->ref) {
        int r = (int)q->ref[idx];
        double fl = floor(u);
        int lower = (int)(fl + z);
        int interior = (lower >= q->qmin) && (lower + 1 <= q->qmax);
        int near = fabs((u - fl) - 0.5) < q->window;
        if (interior && near) {
            if (r == lower || r == lower + 1) {
                code = r;
                q->ties++;
            } else {
                q->mismatches++;
            }
        } else if (r != code) {
            q->mismatches++;
        }
    }
    *u_out = u;
    *c_out = code;
    *v_out = s * ((double)code - z);
}

/* ------------------------------------------------------------------ */
/* BaKron-naive: raster order, one entry at a time, full rank-1 update */
/* (Proposition 3.1).  order 0 = row-major raster, 1 = column-major.   */
/* Both are linear extensions of the product order, so Theorem 3.2     */
/* says they agree.                                                    */
/* ------------------------------------------------------------------ */
int orc_naive(int64_t m, int64_t n, const double *W, const double *LA,
              const double *LB, const double *scales, const double *zeros,
              int kind, int qmin, int qmax, int order,
              const int8_t *ref_codes, double window,
              int32_t *codes, double *V, double *E, double *U,
              int64_t *counts /* [ties, mismatches] */)
{
    double *Wk = (double *)malloc(sizeof(double) * (size_t)(m * n));
    double *LAt = (double *)malloc(sizeof(double) * (size_t)(n * n));
    if (!Wk || !LAt) { free(Wk); free(LAt); return 1; }
    memcpy(Wk, W, sizeof(double) * (size_t)(m * n));
    /* LAt[j][j2] = LA[j2][j]: column j of LA stored contiguously */
    for (int64_t a = 0; a < n; a++)
        for (int64_t b = 0; b < n; b++) LAt[a * n + b] = LA[b * n + a];

    qctx q = {kind, qmin, qmax, ref_codes, window, 0, 0};
    int64_t total = m * n;
    for (int64_t t = 0; t < total; t++) {
        int64_t i = order == 0 ? t / n : t % m;
        int64_t j = order == 0 ? t % n : t / m;
        int64_t idx = i * n + j;
        double P = Wk[idx], u, v;
        int c;
        round_entry(&q, idx, P, scales[i], zeros[i], &u, &c, &v);
        double e = (P - v) / (LB[i * m + i] * LA[j * n + j]);
        codes[idx] = c;
        V[idx] = v;
        E[idx] = e;
        U[idx] = u;
        const double *acol = LAt + j * n;
        int64_t work = (m - i) * (n - j);
#pragma omp parallel for schedule(static) if (work > 65536)
        for (int64_t i2 = i; i2 < m; i2++) {
            double f = e * LB[i2 * m + i];
            double *row = Wk + i2 * n;
            for (int64_t j2 = j; j2 < n; j2++) row[j2] -= f * acol[j2];
        }
    }
    counts[0] = q.ties;
    counts[1] = q.mismatches;
    free(Wk);
    free(LAt);
    return 0;
}

/* ------------------------------------------------------------------ */
/* BaKron-antidiagonal: round a whole anti-diagonal i+j=d from the     */
/* current values, then apply every rank-1 update of that diagonal.    */
/* ------------------------------------------------------------------ */
int orc_antidiag(int64_t m, int64_t n, const double *W, const double *LA,
                 const double *LB, const double *scales, const double *zeros,
                 int kind, int qmin, int qmax, int32_t *codes, double *V,
                 double *E, double *U)
{
    double *Wk = (double *)malloc(sizeof(double) * (size_t)(m * n));
    if (!Wk) return 1;
    memcpy(Wk, W, sizeof(double) * (size_t)(m * n));
    qctx q = {kind, qmin, qmax, NULL, 0.0, 0, 0};
    for (int64_t d = 0; d <= m + n - 2; d++) {
        int64_t ilo = d - (n - 1) > 0 ? d - (n - 1) : 0;
        int64_t ihi = d < m - 1 ? d : m - 1;
        for (int64_t i = ilo; i <= ihi; i++) {
            int64_t j = d - i, idx = i * n + j;
            double P = Wk[idx], u, v;
            int c;
            round_entry(&q, idx, P, scales[i], zeros[i], &u, &c, &v);
            codes[idx] = c;
            V[idx] = v;
            E[idx] = (P - v) / (LB[i * m + i] * LA[j * n + j]);
            U[idx] = u;
        }
        for (int64_t i = ilo; i <= ihi; i++) {
            int64_t j = d - i;
            double e = E[i * n + j];
            for (int64_t i2 = i; i2 < m; i2++) {
                double f = e * LB[i2 * m + i];
                for (int64_t j2 = j; j2 < n; j2++)
                    Wk[i2 * n + j2] -= f * LA[j2 * n + j];
            }
        }
    }
    free(Wk);
    return 0;
}

/* ------------------------------------------------------------------ */
/* BaKron (Algorithm 6, plain reading) at single-diagonal granularity: */
/* solve(k, l) handles diagonals [k, k+l).  A single diagonal is       */
/* rounded in parallel; otherwise split at h = floor(l/2), solve the   */
/* first half, apply the postponed update from S = [k, k+h) to         */
/* R = [k+h, k+l) as two matrix products  W[R] -= (LB (E_S LA^T))[R],  */
/* then solve the second half.                                         */
/* ------------------------------------------------------------------ */
typedef struct {
    int64_t m, n;
    double *Wk, *T;
    const double *LA, *LB, *scales, *zeros;
    int32_t *codes;
    double *V, *E, *U;
    qctx q;
} rctx;

static void rec_solve(rctx *r, int64_t k, int64_t l)
{
    int64_t m = r->m, n = r->n;
    if (l == 1) {
        for (int64_t i = 0; i < m; i++) {
            int64_t j = k - i;
            if (j < 0 || j >= n) continue;
            int64_t idx = i * n + j;
            double P = r->Wk[idx], u, v;
            int c;
            round_entry(&r->q, idx, P, r->scales[i], r->zeros[i], &u, &c, &v);
            r->codes[idx] = c;
            r->V[idx] = v;
            r->E[idx] = (P - v) / (r->LB[i * m + i] * r->LA[j * n + j]);
            r->U[idx] = u;
        }
        return;
    }
    int64_t h = l / 2;
    rec_solve(r, k, h);
    /* T = E_S LA^T  (E masked to the diagonals of S) */
    for (int64_t i = 0; i < m; i++)
        for (int64_t jj = 0; jj < n; jj++) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; j++) {
                int64_t dg = i + j;
                if (dg < k || dg >= k + h) continue;
                acc += r->E[i * n + j] * r->LA[jj * n + j];
            }
            r->T[i * n + jj] = acc;
        }
    /* U = LB T, subtracted on R only */
    for (int64_t i2 = 0; i2 < m; i2++)
        for (int64_t jj = 0; jj < n; jj++) {
            int64_t dg = i2 + jj;
            if (dg < k + h || dg >= k + l) continue;
            double acc = 0.0;
            for (int64_t i = 0; i < m; i++) acc += r->LB[i2 * m + i] * r->T[i * n + jj];
            r->Wk[i2 * n + jj] -= acc;
        }
    rec_solve(r, k + h, l - h);
}

int orc_recursive(int64_t m, int64_t n, const double *W, const double *LA,
                  const double *LB, const double *scales, const double *zeros,
                  int kind, int qmin, int qmax, int32_t *codes, double *V,
                  double *E, double *U)
{
    rctx r;
    r.m = m;
    r.n = n;
    r.Wk = (double *)malloc(sizeof(double) * (size_t)(m * n));
    r.T = (double *)malloc(sizeof(double) * (size_t)(m * n));
    if (!r.Wk || !r.T) { free(r.Wk); free(r.T); return 1; }
    memcpy(r.Wk, W, sizeof(double) * (size_t)(m * n));
    r.LA = LA;
    r.LB = LB;
    r.scales = scales;
    r.zeros = zeros;
    r.codes = codes;
    r.V = V;
    r.E = E;
    r.U = U;
    qctx q = {kind, qmin, qmax, NULL, 0.0, 0, 0};
    r.q = q;
    if (m > 0 && n > 0) rec_solve(&r, 0, m + n - 1);
    free(r.Wk);
    free(r.T);
    return 0;
}
