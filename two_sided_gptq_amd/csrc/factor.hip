// factor.hip -- bakron_factor: L lower with L L^T = H^-1.
//
// The solver consumes the lower Cholesky factors of A^-1 and B^-1 (pith.science
// review of arXiv 2608.06291, "What carries the argument").  Instead of
// inverting H and factoring again, this uses the reverse-order factorisation:
// with J the exchange matrix, let G = J H J = C C^T (ordinary lower Cholesky);
// then H^-1 = J C^-T C^-1 J = (J C^-T J)(J C^-T J)^T and J C^-T J is lower
// triangular with a positive diagonal, so L = J C^-T J, i.e.
// L[a][b] = (C^-1)[d-1-b][d-1-a].
//
// C and X = C^-1 come from one recursion in fp64 (L is rounded to fp32 at the
// end).  For a diagonal block split as [G11 .; G21 G22]:
//   (C11, X11) = recurse(G11)
//   C21  = G21 X11^T                 (the panel solve, as a product)
//   G22 -= C21 C21^T                 (lower tiles only)
//   (C22, X22) = recurse(G22)
//   X21  = -X22 (C21 X11)
// down to 64 x 64 blocks, which one workgroup factors and inverts with the
// block held in registers (base_kernel).  The products run on fp64 MFMA
// (v_mfma_f64_16x16x4f64) in 64 x 64 output tiles, skipping the k blocks where
// a triangular operand is zero.
#include <vector>

#include "common.hpp"

namespace bakron {
namespace {

constexpr int FT = 64;
constexpr int FP = 65;   // LDS row stride (doubles) of the base block
constexpr int GK = 32;   // k chunk of the products
constexpr int GS = GK + 1;

typedef double doublex4 __attribute__((ext_vector_type(4)));

// G (dp x dp) = J H J on the leading d x d block (lower triangle of H read
// only), identity on the padding.
__global__ __launch_bounds__(256) void load_reversed_kernel(const float *__restrict__ H, int64_t d,
                                                            double *__restrict__ G, int64_t dp) {
    const int64_t total = dp * dp;
    for (int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx / dp, j = idx - i * dp;
        double v;
        if (i < d && j < d) {
            const int64_t a = d - 1 - i, b = d - 1 - j;
            v = (double)(a >= b ? H[a * d + b] : H[b * d + a]);
        } else {
            v = (i == j) ? 1.0 : 0.0;
        }
        G[idx] = v;
    }
}

// 1 / sqrt(x) for x > 0: the hardware estimate and two Newton steps, within
// about an ulp of the rounded quotient.
__device__ __forceinline__ double rsqrt_nr(double x) {
    double y = __builtin_amdgcn_rsq(x);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const double h = 0.5 * x * y;
        y = fma(y, fma(-h, y, 0.5), y);
    }
    return y;
}

// One 64 x 64 diagonal block at (off, off): its Cholesky factor and the
// inverse of that factor, right-looking and interleaved, one workgroup.
// Thread (i, q) = (t / 4, t % 4) owns the entries of row i in the columns
// k = q (mod 4), 16 of A (the trailing matrix, then C) and 16 of S (pending
// sums of X = C^-1).  Columns go in groups jb of four; during group jb the
// thread holds, in registers with fixed indices,
//   ar[m'] = A[i][4 (jb + m') + q]   (m' = 0..15; zero past the block)
//   sr[m'] = S[i][4 (jb - m') + q]   (m' = 0..15; zero before the block)
// and between groups both windows move by one (the finished A entry ar[0]
// goes to the LDS staging copy of the block).  At column j = 4 jb + qj:
//   publish  r = 1 / sqrt(A_jj) (from the diagonal's owner), the column
//            A[k][j] unscaled (from its owners, rows k > j), and the pending
//            row S[j][c] with -1 at c = j (from row j's threads)
//   barrier
//   update   the column's owners scale C_ij = A_ij r; every row i > j, with
//            w = A_ij r^2: A_ik -= w A_kj (k > j), i.e. C_ij C_kj, and
//            S_ic -= w S'_jc (c <= j), i.e. + C_ij X_jc with X_jc = -S_jc r
//            (c < j), X_jj = r; row j's threads keep r_j.
// Row j of X is X_jc = -S_jc r_j (c < j), X_jj = r_j, formed when the block is
// written out.  Rows i <= j take w = 0, which leaves them unchanged.  The
// published rows sit in LDS rows of 32 with zero padding on the side the
// windows run past, so only the entries of the current group need a mask.
// Two LDS sets alternate by column parity, so one barrier per column
// separates every write from the reads of the same set.  The block is staged
// through LDS on the way in and out, so the global accesses are coalesced.
__global__ __launch_bounds__(256) void base_kernel(const double *__restrict__ G, double *C, double *X,
                                                   int64_t dp, int64_t off, int32_t *dev_status) {
    constexpr int NM = FT / 4;
    __shared__ double st[FT * FP];          // staging of the block
    // rows of 34 doubles, so the four rows a wave reads start 16 bytes apart in the banks
    constexpr int RW = 2 * NM + 2;
    __shared__ double s_col[2][4][RW];  // [parity][k % 4][k / 4], zero at k / 4 >= 16
    __shared__ double s_xs[2][4][RW];   // [parity][c % 4][16 + c / 4], zero below 16
    __shared__ double s_rc[2];
    const int t = threadIdx.x, ri = t >> 2, q = t & 3;
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int i = idx >> 6, k = idx & 63;
        st[i * FP + k] = k <= i ? G[(off + i) * dp + off + k] : 0.0;
    }
    for (int idx = t; idx < 2 * 4 * RW; idx += 256) {
        (&s_col[0][0][0])[idx] = 0.0;
        (&s_xs[0][0][0])[idx] = 0.0;
    }
    __syncthreads();
    double ar[NM], sr[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        ar[m] = st[ri * FP + 4 * m + q];
        sr[m] = 0.0;
    }
    int bad = 0;
    double rrow = 0.0;  // r_i of this thread's row, once column i is done
    for (int jb = 0; jb < NM; ++jb) {
        if (jb > 0) {
            st[ri * FP + 4 * (jb - 1) + q] = ar[0];
#pragma unroll
            for (int m = 0; m + 1 < NM; ++m) ar[m] = ar[m + 1];
            ar[NM - 1] = 0.0;
#pragma unroll
            for (int m = NM - 1; m > 0; --m) sr[m] = sr[m - 1];
            sr[0] = 0.0;
        }
#pragma unroll
        for (int qj = 0; qj < 4; ++qj) {
            const int j = 4 * jb + qj, par = qj & 1;
            // publish
            if (ri == j && q == qj) {
                double ajj = ar[0];
                if (!(ajj > 0.0) || !isfinite(ajj)) {
                    bad = 1;
                    ajj = 1.0;
                }
                s_rc[par] = rsqrt_nr(ajj);
            }
            if (q == qj && ri > j) s_col[par][ri & 3][ri >> 2] = ar[0];
            if (ri == j) {
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    s_xs[par][q][NM + jb - m] = (m == 0 && q == qj) ? -1.0 : sr[m];
            }
            __syncthreads();
            // update
            const double rc = s_rc[par];
            rrow = ri == j ? rc : rrow;
            const double w = ri > j ? s_col[par][ri & 3][ri >> 2] * rc * rc : 0.0;
            const double *cq = &s_col[par][q][jb];
            const double *xq = &s_xs[par][q][NM + jb];
            {   // the current group: column 4 jb + q is past j for q > qj, j itself for q = qj
                const double v = fma(-w, cq[0], ar[0]);
                const double sc = ri > j ? ar[0] * rc : ar[0];
                ar[0] = q > qj ? v : (q == qj ? sc : ar[0]);
                const double u = fma(-w, xq[0], sr[0]);
                sr[0] = q <= qj ? u : sr[0];
            }
#pragma unroll
            for (int m = 1; m < NM; ++m) {
                ar[m] = fma(-w, cq[m], ar[m]);
                sr[m] = fma(-w, xq[-m], sr[m]);
            }
        }
    }
    // C (upper part zero, diagonal sqrt of the last A_ii) and X through LDS
    st[ri * FP + 4 * (NM - 1) + q] = ar[0];
    __syncthreads();
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int i = idx >> 6, k = idx & 63;
        const double v = st[i * FP + k];
        C[(off + i) * dp + off + k] = k < i ? v : (k == i ? sqrt(v) : 0.0);
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NM; ++m) {
        const int k = 4 * (NM - 1 - m) + q;
        st[ri * FP + k] = k < ri ? -sr[m] * rrow : (k == ri ? rrow : 0.0);
    }
    __syncthreads();
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int i = idx >> 6, k = idx & 63;
        X[(off + i) * dp + off + k] = st[i * FP + k];
    }
    if (bad && dev_status) atomicOr(dev_status, BAKRON_DEV_NOT_PD);
}

// C (M x N) = beta C + alpha sum_k A[i][k] op(B)[k][j], op(B)[k][j] = B[j][k]
// (bnn = 0) or B[k][j] (bnn = 1); M, N, K multiples of 64.  kmode skips k
// blocks where a triangular operand is zero: 1 A lower (k < 64 (ib+1)), 2 the
// B rows lower (k < 64 (jb+1), bnn = 0), 3 B lower (k >= 64 jb, bnn = 1).  lower:
// only the output tiles on or below the diagonal (grid.x enumerates them).
struct DGemm {
    const double *A;
    int64_t lda;
    const double *B;
    int64_t ldb;
    double *C;
    int64_t ldc;
    int M, N, K, bnn, kmode, lower;
    double alpha, beta;
};

__global__ __launch_bounds__(256) void dgemm_kernel(DGemm g) {
    int ib, jb;
    if (g.lower) {
        const int64_t x = blockIdx.x;
        int64_t a = (int64_t)((sqrt(8.0 * (double)x + 1.0) - 1.0) * 0.5);
        while (a * (a + 1) / 2 > x) --a;
        while ((a + 1) * (a + 2) / 2 <= x) ++a;
        ib = (int)a;
        jb = (int)(x - a * (a + 1) / 2);
    } else {
        ib = blockIdx.y;
        jb = blockIdx.x;
    }
    int klo = 0, khi = g.K;
    if (g.kmode == 1) khi = min(g.K, FT * (ib + 1));
    if (g.kmode == 2) khi = min(g.K, FT * (jb + 1));
    if (g.kmode == 3) klo = FT * jb;
    __shared__ double As[FT * GS];
    __shared__ double Bs[FT * GS];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int qr = w >> 1, qc = w & 1;
    doublex4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = doublex4{0.0, 0.0, 0.0, 0.0};
    // Each thread moves 8 consecutive doubles of A and of B per k chunk: A and
    // (bnn = 0) B by row (row t / 4, k offset 8 (t % 4)); B (bnn = 1) by k row
    // (t / 8, columns 8 (t % 8) ..).  The next chunk is read into registers
    // while the current one is multiplied.
    const int row = t >> 2, kk = (t & 3) * 8;
    const int kr = t >> 3, jj = (t & 7) * 8;
    const double *Asrc = g.A + ((int64_t)FT * ib + row) * g.lda + kk;
    const double *Bsrc = g.bnn ? g.B + (int64_t)kr * g.ldb + (int64_t)FT * jb + jj
                               : g.B + ((int64_t)FT * jb + row) * g.ldb + kk;
    const int64_t bstep = g.bnn ? (int64_t)g.ldb : 1;  // B address advance per unit of k
    double ra[8], rb[8];
    if (klo < khi) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            ra[q] = Asrc[klo + q];
            rb[q] = Bsrc[klo * bstep + q];
        }
    }
    for (int k0 = klo; k0 < khi; k0 += GK) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 8; ++q) As[row * GS + kk + q] = ra[q];
        if (!g.bnn) {
#pragma unroll
            for (int q = 0; q < 8; ++q) Bs[row * GS + kk + q] = rb[q];
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) Bs[(jj + q) * GS + kr] = rb[q];
        }
        __syncthreads();
        if (k0 + GK < khi) {
            const int kn = k0 + GK;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                ra[q] = Asrc[kn + q];
                rb[q] = Bsrc[kn * bstep + q];
            }
        }
        // lane l supplies A[l % 16][k] and B[k][l % 16] with k = 4 s + l / 16
#pragma unroll
        for (int s = 0; s < GK / 4; ++s) {
            double av[2], bv[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) av[a] = As[(32 * qr + 16 * a + (lane & 15)) * GS + 4 * s + (lane >> 4)];
#pragma unroll
            for (int b = 0; b < 2; ++b) bv[b] = Bs[(32 * qc + 16 * b + (lane & 15)) * GS + 4 * s + (lane >> 4)];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    }
    // register v of lane l holds D[l / 16 + 4 v][l % 16] of each 16 x 16 block
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = (int64_t)FT * ib + 32 * qr + 16 * a + (lane >> 4) + 4 * v;
                const int64_t col = (int64_t)FT * jb + 32 * qc + 16 * b + (lane & 15);
                double *c = g.C + row * g.ldc + col;
                const double r = g.alpha * acc[a][b][v];
                *c = g.beta != 0.0 ? fma(g.beta, *c, r) : r;
            }
}

// L[a][b] = X[d-1-b][d-1-a] for b <= a, 0 above; tiled transpose through LDS
__global__ __launch_bounds__(256) void write_l_kernel(const double *X, int64_t dp, int64_t d, float *L) {
    __shared__ float T[FT * (FT + 1)];
    const int64_t a0 = (int64_t)blockIdx.y * FT, b0 = (int64_t)blockIdx.x * FT;
    const int t = threadIdx.x;
    // source rows d-1-b (b in [b0, b0+64)), columns d-1-a (a in [a0, a0+64))
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int bb = idx / FT, aa = idx % FT;  // consecutive threads: consecutive a
        const int64_t a = a0 + aa, b = b0 + bb;
        float v = 0.0f;
        if (a < d && b < d && b <= a) v = (float)X[(d - 1 - b) * dp + (d - 1 - a)];
        T[aa * (FT + 1) + bb] = v;
    }
    __syncthreads();
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int aa = idx / FT, bb = idx % FT;
        const int64_t a = a0 + aa, b = b0 + bb;
        if (a < d && b < d) L[a * d + b] = T[aa * (FT + 1) + bb];
    }
}

struct FBufs {
    double *G, *C, *X, *T;
};

size_t fcarve(void *ws, int64_t dp, FBufs *f) {
    Carver cv(ws);
    double *G = cv.take<double>(dp * dp);
    double *C = cv.take<double>(dp * dp);
    double *X = cv.take<double>(dp * dp);
    double *T = cv.take<double>(dp * dp);
    if (f) *f = FBufs{G, C, X, T};
    return cv.used;
}

struct Factor {
    FBufs f;
    int64_t dp;
    int32_t *dev_status;
    hipStream_t stream;
};

int32_t gemm(const Factor &fc, const double *A, const double *B, double *Cout, int M, int N, int K,
             int bnn, int kmode, int lower, double alpha, double beta) {
    DGemm g{A, fc.dp, B, fc.dp, Cout, fc.dp, M, N, K, bnn, kmode, lower, alpha, beta};
    const int mb = M / FT, nb = N / FT;
    if (lower) {
        hipLaunchKernelGGL(dgemm_kernel, dim3((unsigned)(mb * (mb + 1) / 2)), dim3(256), 0, fc.stream, g);
    } else {
        hipLaunchKernelGGL(dgemm_kernel, dim3(nb, mb), dim3(256), 0, fc.stream, g);
    }
    BK_LAUNCH_CHECK("dgemm_kernel");
    return BAKRON_OK;
}

// factor and invert the diagonal block [off, off + n) of G into C and X
int32_t recurse(const Factor &fc, int64_t off, int64_t n) {
    const int64_t dp = fc.dp;
    if (n == FT) {
        hipLaunchKernelGGL(base_kernel, dim3(1), dim3(256), 0, fc.stream, fc.f.G, fc.f.C, fc.f.X, dp,
                           off, fc.dev_status);
        BK_LAUNCH_CHECK("base_kernel");
        return BAKRON_OK;
    }
    const int64_t n1 = (n / FT / 2) * FT, n2 = n - n1;
    int32_t st = recurse(fc, off, n1);
    if (st != BAKRON_OK) return st;
    auto at = [dp](double *p, int64_t r, int64_t c) { return p + r * dp + c; };
    double *G = fc.f.G, *C = fc.f.C, *X = fc.f.X, *T = fc.f.T;
    // C21 = G21 X11^T (X11 lower: the rows of X11 end at the output column block)
    st = gemm(fc, at(G, off + n1, off), at(X, off, off), at(C, off + n1, off), (int)n2, (int)n1,
              (int)n1, 0, 2, 0, 1.0, 0.0);
    if (st != BAKRON_OK) return st;
    // G22 -= C21 C21^T, lower tiles
    st = gemm(fc, at(C, off + n1, off), at(C, off + n1, off), at(G, off + n1, off + n1), (int)n2,
              (int)n2, (int)n1, 0, 0, 1, -1.0, 1.0);
    if (st != BAKRON_OK) return st;
    st = recurse(fc, off + n1, n2);
    if (st != BAKRON_OK) return st;
    // T = C21 X11 (X11 lower: rows k >= the output column block), X21 = -X22 T (X22 lower)
    st = gemm(fc, at(C, off + n1, off), at(X, off, off), at(T, off + n1, off), (int)n2, (int)n1,
              (int)n1, 1, 3, 0, 1.0, 0.0);
    if (st != BAKRON_OK) return st;
    st = gemm(fc, at(X, off + n1, off + n1), at(T, off + n1, off), at(X, off + n1, off), (int)n2,
              (int)n1, (int)n2, 1, 1, 0, -1.0, 0.0);
    return st;
}

}  // namespace
}  // namespace bakron

using namespace bakron;

extern "C" size_t bakron_factor_workspace_size(int64_t d) {
    if (d < 1 || d > (int64_t(1) << 17)) return 0;
    return fcarve(reinterpret_cast<void *>(256), round_up(d, FT), nullptr);
}

extern "C" int32_t bakron_factor(const float *H, int64_t d, float *L, int32_t *dev_status, void *ws,
                                 size_t ws_bytes, void *stream_) {
    clear_error();
    BK_REQUIRE(H && L, "H and L must be non-NULL");
    BK_REQUIRE(d >= 1 && d <= (int64_t(1) << 17), "bad size d=%lld", (long long)d);
    const size_t need = bakron_factor_workspace_size(d);
    if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) {
        set_error("workspace needs %zu bytes at 256-byte alignment (got %zu at %p)", need,
                  ws_bytes, ws);
        return BAKRON_ERR_WORKSPACE;
    }
    int32_t st = check_device();
    if (st != BAKRON_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    Factor fc;
    fc.dp = round_up(d, FT);
    fc.dev_status = dev_status;
    fc.stream = stream;
    fcarve(ws, fc.dp, &fc.f);
    hipLaunchKernelGGL(load_reversed_kernel, dim3(2048), dim3(256), 0, stream, H, d, fc.f.G, fc.dp);
    BK_LAUNCH_CHECK("load_reversed_kernel");
    st = recurse(fc, 0, fc.dp);
    if (st != BAKRON_OK) return st;
    const unsigned tl = (unsigned)((d + FT - 1) / FT);
    hipLaunchKernelGGL(write_l_kernel, dim3(tl, tl), dim3(256), 0, stream, fc.f.X, fc.dp, d, L);
    BK_LAUNCH_CHECK("write_l_kernel");
    return BAKRON_OK;
}
