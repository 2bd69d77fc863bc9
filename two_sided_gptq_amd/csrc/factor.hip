// factor.hip -- bakron_factor: L lower with L L^T = H^-1.
//
// The solver consumes the lower Cholesky factors of A^-1 and B^-1 (pith.science
// review of arXiv 2608.06291, "What carries the argument").  Instead of
// inverting H and factoring again, this uses the reverse-order factorisation:
// with J the exchange matrix, let G = J H J = C C^T (ordinary lower Cholesky);
// then H^-1 = J C^-T C^-1 J = (J C^-T J)(J C^-T J)^T and J C^-T J is lower
// triangular with a positive diagonal, so L = J C^-T J, i.e.
// L[a][b] = (C^-1)[d-1-b][d-1-a].  One Cholesky and one triangular inverse,
// both blocked in 64 x 64 tiles and computed in fp64; L is rounded to fp32.
#include "common.hpp"

namespace bakron {
namespace {

constexpr int FT = 64;
constexpr int FP = 65;  // LDS row stride (doubles) for in-block solves
constexpr int KC = 16;  // K chunk of the tile products

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

// unblocked Cholesky of the diagonal block (kb, kb), in place, upper part zeroed
__global__ __launch_bounds__(256) void chol_diag_kernel(double *G, int64_t dp, int kb,
                                                        int32_t *dev_status) {
    __shared__ double A[FT * FP];
    __shared__ int s_bad;
    const int t = threadIdx.x;
    double *blk = G + (int64_t)kb * FT * dp + (int64_t)kb * FT;
    for (int idx = t; idx < FT * FT; idx += 256) A[(idx / FT) * FP + idx % FT] = blk[(idx / FT) * dp + idx % FT];
    if (t == 0) s_bad = 0;
    __syncthreads();
    for (int j = 0; j < FT; ++j) {
        if (t == 0) {
            double v = A[j * FP + j];
            if (!(v > 0.0) || !isfinite(v)) {
                s_bad = 1;
                v = 1.0;
            }
            A[j * FP + j] = sqrt(v);
        }
        __syncthreads();
        if (t > j && t < FT) A[t * FP + j] /= A[j * FP + j];
        __syncthreads();
        for (int idx = t; idx < FT * FT; idx += 256) {
            const int i = idx / FT, k = idx % FT;
            if (k > j && k <= i) A[i * FP + k] -= A[i * FP + j] * A[k * FP + j];
        }
        __syncthreads();
    }
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int i = idx / FT, k = idx % FT;
        blk[i * dp + k] = (k <= i) ? A[i * FP + k] : 0.0;
    }
    if (t == 0 && s_bad && dev_status) atomicOr(dev_status, BAKRON_DEV_NOT_PD);
}

// panel below the diagonal block: G[ib][kb] <- G[ib][kb] C^-T, C = G[kb][kb]
__global__ __launch_bounds__(64) void trsm_panel_kernel(double *G, int64_t dp, int kb) {
    __shared__ double C[FT * FP];
    __shared__ double X[FT * FP];
    const int t = threadIdx.x;
    const int ib = kb + 1 + blockIdx.x;
    const double *cblk = G + (int64_t)kb * FT * dp + (int64_t)kb * FT;
    double *xblk = G + (int64_t)ib * FT * dp + (int64_t)kb * FT;
    for (int idx = t; idx < FT * FT; idx += 64) {
        C[(idx / FT) * FP + idx % FT] = cblk[(idx / FT) * dp + idx % FT];
        X[(idx / FT) * FP + idx % FT] = xblk[(idx / FT) * dp + idx % FT];
    }
    __syncthreads();
    // row t: x C^T = b  ->  x_j = (b_j - sum_{k<j} x_k C[j][k]) / C[j][j]
    for (int j = 0; j < FT; ++j) {
        double s = X[t * FP + j];
        for (int k = 0; k < j; ++k) s -= X[t * FP + k] * C[j * FP + k];
        X[t * FP + j] = s / C[j * FP + j];
    }
    __syncthreads();
    for (int idx = t; idx < FT * FT; idx += 64) xblk[(idx / FT) * dp + idx % FT] = X[(idx / FT) * FP + idx % FT];
}

// acc (4 x 4 per thread of a 64 x 64 tile) += A(64 x kdim) . op(B), where
// op(B)[k][c] = B[c][k] (b_trans) or B[k][c]
__device__ void tile_mac(const double *A, int64_t lda, const double *B, int64_t ldb, bool b_trans,
                         int kdim, double acc[4][4], double *sA, double *sB) {
    const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
    for (int k0 = 0; k0 < kdim; k0 += KC) {
        __syncthreads();
        for (int idx = t; idx < FT * KC; idx += 256) {
            const int r = idx / KC, kk = idx % KC;
            sA[r * (KC + 1) + kk] = A[(int64_t)r * lda + k0 + kk];
            if (b_trans) {
                sB[r * (KC + 1) + kk] = B[(int64_t)r * ldb + k0 + kk];
            } else {
                const int kk2 = idx / FT, c = idx % FT;
                sB[c * (KC + 1) + kk2] = B[(int64_t)(k0 + kk2) * ldb + c];
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int kk = 0; kk < KC; ++kk) {
            double a[4], b[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a[q] = sA[(ty * 4 + q) * (KC + 1) + kk];
                b[q] = sB[(tx * 4 + q) * (KC + 1) + kk];
            }
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[p][q] = fma(a[p], b[q], acc[p][q]);
        }
    }
}

// trailing update G[ib][jb] -= G[ib][kb] G[jb][kb]^T for kb < jb <= ib < Nb
__global__ __launch_bounds__(256) void syrk_update_kernel(double *G, int64_t dp, int kb, int Nb) {
    __shared__ double sA[FT * (KC + 1)];
    __shared__ double sB[FT * (KC + 1)];
    const int64_t x = blockIdx.x;
    int64_t a = (int64_t)((sqrt(8.0 * (double)x + 1.0) - 1.0) * 0.5);
    while (a * (a + 1) / 2 > x) --a;
    while ((a + 1) * (a + 2) / 2 <= x) ++a;
    const int ib = kb + 1 + (int)a;
    const int jb = kb + 1 + (int)(x - a * (a + 1) / 2);
    if (ib >= Nb || jb > ib) return;
    double acc[4][4] = {};
    tile_mac(G + (int64_t)ib * FT * dp + (int64_t)kb * FT, dp, G + (int64_t)jb * FT * dp + (int64_t)kb * FT,
             dp, true, FT, acc, sA, sB);
    const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
    double *c = G + (int64_t)ib * FT * dp + (int64_t)jb * FT;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) c[(int64_t)(ty * 4 + p) * dp + tx * 4 + q] -= acc[p][q];
}

// inverse of every diagonal block of the lower factor C: Dinv[b] = C[b][b]^-1,
// also written to X[b][b]
__global__ __launch_bounds__(64) void trinv_diag_kernel(const double *C, int64_t dp, double *X,
                                                        double *Dinv) {
    __shared__ double Cs[FT * FP];
    __shared__ double Y[FT * FP];
    const int t = threadIdx.x, b = blockIdx.x;
    const double *cblk = C + (int64_t)b * FT * dp + (int64_t)b * FT;
    for (int idx = t; idx < FT * FT; idx += 64) Cs[(idx / FT) * FP + idx % FT] = cblk[(idx / FT) * dp + idx % FT];
    __syncthreads();
    // column t of Y = C^-1: forward substitution on e_t
    for (int r = 0; r < FT; ++r) {
        double s = (r == t) ? 1.0 : 0.0;
        for (int k = 0; k < r; ++k) s -= Cs[r * FP + k] * Y[k * FP + t];
        Y[r * FP + t] = s / Cs[r * FP + r];
    }
    __syncthreads();
    double *xblk = X + (int64_t)b * FT * dp + (int64_t)b * FT;
    double *dblk = Dinv + (int64_t)b * FT * FT;
    for (int idx = t; idx < FT * FT; idx += 64) {
        const double v = Y[(idx / FT) * FP + idx % FT];
        xblk[(idx / FT) * dp + idx % FT] = v;
        dblk[idx] = v;
    }
}

// block row i of X = C^-1: X[i][j] = -Dinv[i] sum_{k=j}^{i-1} C[i][k] X[k][j], j < i
__global__ __launch_bounds__(256) void trinv_row_kernel(const double *C, int64_t dp, double *X,
                                                        const double *Dinv, int i) {
    __shared__ double sA[FT * (KC + 1)];
    __shared__ double sB[FT * (KC + 1)];
    __shared__ double R[FT * FP];
    const int j = blockIdx.x;
    const int t = threadIdx.x, ty = t >> 4, tx = t & 15;
    double acc[4][4] = {};
    tile_mac(C + (int64_t)i * FT * dp + (int64_t)j * FT, dp, X + (int64_t)j * FT * dp + (int64_t)j * FT, dp,
             false, (i - j) * FT, acc, sA, sB);
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) R[(ty * 4 + p) * FP + tx * 4 + q] = acc[p][q];
    __syncthreads();
    double out[4][4] = {};
    const double *D = Dinv + (int64_t)i * FT * FT;
    for (int k = 0; k < FT; ++k) {
        double a[4], b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            a[q] = D[(ty * 4 + q) * FT + k];
            b[q] = R[k * FP + tx * 4 + q];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int q = 0; q < 4; ++q) out[p][q] = fma(a[p], b[q], out[p][q]);
    }
    double *xblk = X + (int64_t)i * FT * dp + (int64_t)j * FT;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) xblk[(int64_t)(ty * 4 + p) * dp + tx * 4 + q] = -out[p][q];
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
    double *G, *X, *Dinv;
};

size_t fcarve(void *ws, int64_t dp, FBufs *f) {
    Carver cv(ws);
    double *G = cv.take<double>(dp * dp);
    double *X = cv.take<double>(dp * dp);
    double *D = cv.take<double>(dp * FT);
    if (f) *f = FBufs{G, X, D};
    return cv.used;
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
    const int64_t dp = round_up(d, FT);
    const int Nb = (int)(dp / FT);
    FBufs f;
    fcarve(ws, dp, &f);
    hipLaunchKernelGGL(load_reversed_kernel, dim3(2048), dim3(256), 0, stream, H, d, f.G, dp);
    BK_LAUNCH_CHECK("load_reversed_kernel");
    for (int kb = 0; kb < Nb; ++kb) {
        hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, stream, f.G, dp, kb, dev_status);
        BK_LAUNCH_CHECK("chol_diag_kernel");
        const int below = Nb - kb - 1;
        if (below > 0) {
            hipLaunchKernelGGL(trsm_panel_kernel, dim3(below), dim3(64), 0, stream, f.G, dp, kb);
            BK_LAUNCH_CHECK("trsm_panel_kernel");
            const int64_t tiles = (int64_t)below * (below + 1) / 2;
            hipLaunchKernelGGL(syrk_update_kernel, dim3((unsigned)tiles), dim3(256), 0, stream, f.G, dp,
                               kb, Nb);
            BK_LAUNCH_CHECK("syrk_update_kernel");
        }
    }
    // C^-1, block row by block row
    hipLaunchKernelGGL(trinv_diag_kernel, dim3(Nb), dim3(64), 0, stream, f.G, dp, f.X, f.Dinv);
    BK_LAUNCH_CHECK("trinv_diag_kernel");
    for (int i = 1; i < Nb; ++i) {
        hipLaunchKernelGGL(trinv_row_kernel, dim3(i), dim3(256), 0, stream, f.G, dp, f.X, f.Dinv, i);
        BK_LAUNCH_CHECK("trinv_row_kernel");
    }
    const unsigned tl = (unsigned)((d + FT - 1) / FT);
    hipLaunchKernelGGL(write_l_kernel, dim3(tl, tl), dim3(256), 0, stream, f.X, dp, d, L);
    BK_LAUNCH_CHECK("write_l_kernel");
    return BAKRON_OK;
}
