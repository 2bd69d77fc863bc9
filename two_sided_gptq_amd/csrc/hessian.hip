// hessian.hip -- bakron_hessian: H = X^T X / N + damp_rel * mean(diag) * I.
//
// Kronecker factors from samples with Gram regularisation by a multiple of the
// mean diagonal (pith.science review of arXiv 2608.06291, free parameters).
//
// H is symmetric, so only the 64 x 64 tiles on and below the diagonal are
// computed (the SYRK half of the product) and each off-diagonal tile is also
// stored into its mirrored place.  A tile runs on the fp32 matrix cores
// (v_mfma_f32_32x32x2_f32), 4 waves with one 32 x 32 quadrant each, 64
// samples per K step.  X is read row by row (64 consecutive samples per K step,
// so the tiles at one K step share one contiguous stretch of X) and transposed
// into LDS so that every lane reads its MFMA operands as contiguous float4.
#include "common.hpp"

namespace bakron {
namespace {

constexpr int HT = 64;
constexpr int HP = 68;  // LDS row stride (floats)

typedef float floatx16 __attribute__((ext_vector_type(16)));

// Workgroup x computes the lower-triangle tile (ib, jb) with
// ib (ib + 1) / 2 + jb = x.
__global__ __launch_bounds__(256) void syrk_kernel(const float *__restrict__ X, int64_t N,
                                                   int64_t d, float inv_n, float *__restrict__ H,
                                                   int vec_ok) {
    const int64_t t = blockIdx.x;
    int64_t a = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while (a * (a + 1) / 2 > t) --a;
    while ((a + 1) * (a + 2) / 2 <= t) ++a;
    const int64_t i0 = a * HT, j0 = (t - a * (a + 1) / 2) * HT;
    __shared__ __align__(16) float As[HT * HP];  // As[i][k] = X[k0 + k][i0 + i]
    __shared__ __align__(16) float Bs[HT * HP];  // Bs[j][k] = X[k0 + k][j0 + j]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr = w >> 1, wc = w & 1;
    const int lk = tid >> 4, l4 = (tid & 15) * 4;
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    const float *ap = As + (wr * 32 + (lane & 31)) * HP + 32 * (lane >> 5);
    const float *bp = Bs + (wc * 32 + (lane & 31)) * HP + 32 * (lane >> 5);
    for (int64_t k0 = 0; k0 < N; k0 += HT) {
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t k = k0 + lk + 16 * p;
            float xa[4], xb[4];
            const bool full = vec_ok && k < N && i0 + l4 + 3 < d && j0 + l4 + 3 < d;
            if (full) {
                const float4 va = *reinterpret_cast<const float4 *>(X + k * d + i0 + l4);
                const float4 vb = *reinterpret_cast<const float4 *>(X + k * d + j0 + l4);
                xa[0] = va.x; xa[1] = va.y; xa[2] = va.z; xa[3] = va.w;
                xb[0] = vb.x; xb[1] = vb.y; xb[2] = vb.z; xb[3] = vb.w;
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xa[q] = (k < N && i0 + l4 + q < d) ? X[k * d + i0 + l4 + q] : 0.0f;
                    xb[q] = (k < N && j0 + l4 + q < d) ? X[k * d + j0 + l4 + q] : 0.0f;
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                As[(l4 + q) * HP + lk + 16 * p] = xa[q];
                Bs[(l4 + q) * HP + lk + 16 * p] = xb[q];
            }
        }
        __syncthreads();
#pragma unroll
        for (int s4 = 0; s4 < 8; ++s4) {
            const float4 av = *reinterpret_cast<const float4 *>(ap + 4 * s4);
            const float4 bv = *reinterpret_cast<const float4 *>(bp + 4 * s4);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv.w, acc, 0, 0, 0);
        }
    }
    // accumulator: lane l holds column l % 32 of its quadrant, register v row
    // 8 (v / 4) + 4 (l / 32) + v % 4.  The tile goes to H directly; its mirror
    // goes through LDS so that both stores write rows.
    const int col = wc * 32 + (lane & 31);
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = wr * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const float val = acc[v] * inv_n;
        As[row * HP + col] = val;
        const int64_t gi = i0 + row, gj = j0 + col;
        if (gi < d && gj < d) H[gi * d + gj] = val;
    }
    if (i0 == j0) return;  // a diagonal tile is its own mirror
    __syncthreads();
    for (int idx = tid; idx < HT * HT; idx += 256) {
        const int r = idx >> 6, c = idx & 63;  // H[j0 + r][i0 + c] = tile[c][r]
        const int64_t gi = j0 + r, gj = i0 + c;
        if (gi < d && gj < d) H[gi * d + gj] = As[c * HP + r];
    }
}

// mean of the diagonal in a fixed order, then H_ii += damp_rel * mean
__global__ __launch_bounds__(256) void damp_kernel(float *H, int64_t d, float damp_rel) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < d; i += 256) s += (double)H[i * d + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    const float add = (float)((double)damp_rel * (red[0] / (double)d));
    for (int64_t i = threadIdx.x; i < d; i += 256) H[i * d + i] += add;
}

constexpr int64_t MAX_D = int64_t(1) << 20;
constexpr int64_t MAX_N = int64_t(1) << 40;

}  // namespace
}  // namespace bakron

using namespace bakron;

extern "C" size_t bakron_hessian_workspace_size(int64_t N, int64_t d) {
    (void)N;
    (void)d;
    return 0;
}

extern "C" int32_t bakron_hessian(const float *X, int64_t N, int64_t d, float damp_rel, float *H,
                                  void *ws, size_t ws_bytes, void *stream_) {
    clear_error();
    BK_REQUIRE(X && H, "X and H must be non-NULL");
    BK_REQUIRE(N >= 1 && d >= 1 && d <= MAX_D && N <= MAX_N, "bad sizes N=%lld d=%lld",
               (long long)N, (long long)d);
    BK_REQUIRE(damp_rel >= 0.0f && damp_rel < INFINITY, "damp_rel must be finite and >= 0");
    (void)ws;
    (void)ws_bytes;
    int32_t st = check_device();
    if (st != BAKRON_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int64_t tiles = (d + HT - 1) / HT;
    const int vec_ok = (d % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    hipLaunchKernelGGL(syrk_kernel, dim3((unsigned)(tiles * (tiles + 1) / 2)), dim3(256), 0, stream, X,
                       N, d, (float)(1.0 / (double)N), H, vec_ok);
    BK_LAUNCH_CHECK("syrk_kernel");
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, stream, H, d, damp_rel);
    BK_LAUNCH_CHECK("damp_kernel");
    return BAKRON_OK;
}
