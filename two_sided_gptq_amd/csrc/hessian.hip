// hessian.hip -- bakron_hessian: H = X^T X / N + damp_rel * mean(diag) * I.
//
// Kronecker factors from samples with Gram regularisation by a multiple of the
// mean diagonal (pith.science review of arXiv 2608.06291, free parameters).
// The Gram product runs on the fp32 matrix cores (v_mfma_f32_32x32x2_f32),
// one 64 x 64 output tile per workgroup, 64 samples per K step; X is read
// row by row (coalesced) and transposed into LDS so that every lane reads its
// MFMA operands as contiguous float4.
#include "common.hpp"

namespace bakron {
namespace {

constexpr int HT = 64;
constexpr int HP = 68;

typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void gram_kernel(const float *__restrict__ X, int64_t N,
                                                   int64_t d, float inv_n, float *__restrict__ H,
                                                   int vec_ok) {
    __shared__ __align__(16) float As[HT * HP];  // As[i][k] = X[k0 + k][i0 + i]
    __shared__ __align__(16) float Bs[HT * HP];  // Bs[j][k] = X[k0 + k][j0 + j]
    const int64_t i0 = (int64_t)blockIdx.y * HT, j0 = (int64_t)blockIdx.x * HT;
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
                const float4 a = *reinterpret_cast<const float4 *>(X + k * d + i0 + l4);
                const float4 b = *reinterpret_cast<const float4 *>(X + k * d + j0 + l4);
                xa[0] = a.x; xa[1] = a.y; xa[2] = a.z; xa[3] = a.w;
                xb[0] = b.x; xb[1] = b.y; xb[2] = b.z; xb[3] = b.w;
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
    const int col = lane & 31;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t gi = i0 + wr * 32 + row, gj = j0 + wc * 32 + col;
        if (gi < d && gj < d) H[gi * d + gj] = acc[v] * inv_n;
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
    (void)ws;
    (void)ws_bytes;
    BK_REQUIRE(X && H, "X and H must be non-NULL");
    BK_REQUIRE(N >= 1 && d >= 1 && d <= (int64_t(1) << 20) && N <= (int64_t(1) << 40),
               "bad sizes N=%lld d=%lld", (long long)N, (long long)d);
    BK_REQUIRE(damp_rel >= 0.0f && damp_rel < INFINITY, "damp_rel must be finite and >= 0");
    int32_t st = check_device();
    if (st != BAKRON_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int tiles = (int)((d + HT - 1) / HT);
    const int vec_ok = (d % 4 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
    hipLaunchKernelGGL(gram_kernel, dim3(tiles, tiles), dim3(256), 0, stream, X, N, d,
                       (float)(1.0 / (double)N), H, vec_ok);
    BK_LAUNCH_CHECK("gram_kernel");
    hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(256), 0, stream, H, d, damp_rel);
    BK_LAUNCH_CHECK("damp_kernel");
    return BAKRON_OK;
}
