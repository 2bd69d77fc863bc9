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
// A 128 x 128 node runs whole in one workgroup (node128_kernel); its 64 x 64
// diagonal blocks are factored and inverted blocked by 16 (base_block).  The
// products run on fp64 MFMA (v_mfma_f64_16x16x4f64) in 64 x 64 or 32 x 32
// output tiles, skipping the k blocks where a triangular operand is zero; the
// wide nodes' T = C21 X11 runs on a side stream beside the recursion into G22.
#include <map>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace bakron {
namespace {

constexpr int FT = 64;
constexpr int FP = 65;   // LDS row stride (doubles) of the base block
constexpr int DB = 16;   // diagonal sub-block of the base

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

__device__ __forceinline__ double readlane_d(const double x, const int lane) {
    const long long b = __double_as_longlong(x);
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)b, lane);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(b >> 32), lane);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// keeps the wave's LDS accesses in program order (the hardware runs one
// wave's LDS operations in order)
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// One 16 x 16 x 16 product on the matrix cores, one wave:
// acc += sa * A B with A[r][k] = pa[r * lda + k], B[k][c] = pb[k * sbk + c * sbc].
// Lane l supplies A[l % 16][k] and B[k][l % 16] for k = 4 s + l / 16; register
// v of lane l holds the output entry (l / 16 + 4 v, l % 16).
__device__ __forceinline__ void mm16(doublex4 &acc, const double *pa, const int lda, const double *pb,
                                     const int sbk, const int sbc, const double sa, const int l) {
    const int r = l & 15, kq = l >> 4;
    double av[4], bv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        av[s] = sa * pa[r * lda + 4 * s + kq];
        bv[s] = pb[(4 * s + kq) * sbk + r * sbc];
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av[s], bv[s], acc, 0, 0, 0);
}

__device__ __forceinline__ doublex4 ld16(const double *p, const int l) {
    doublex4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = p[((l >> 4) + 4 * k) * FP + (l & 15)];
    return v;
}

__device__ __forceinline__ void st16(double *p, const int l, const doublex4 v) {
#pragma unroll
    for (int k = 0; k < 4; ++k) p[((l >> 4) + 4 * k) * FP + (l & 15)] = v[k];
}

// The 16 x 16 diagonal block at (o, o) of sA: its Cholesky factor in place and
// the inverse of that factor into sX, by one wave, right-looking and
// interleaved as for a whole block, with the column exchange through a
// wave-local LDS area (no barrier).  Lane l = 4 i + q holds A[i][4 v + q] and
// S[i][4 v + q] (v = 0..3).  At column j:
//   the pivot's 1 / sqrt r and value come from lane 4 j + j % 4 (readlane);
//   the owners of column j publish P_i = A_ij for rows i > j and zero for rows
//   <= j, and row j's lanes publish S'_jc = S_jc (c < j), -1 (c = j), 0 (c > j),
//   both at position (k % 4) * 4 + k / 4 so each lane reads its four columns
//   as one contiguous run;
//   every entry takes A_ik -= w_i P_k and S_ik -= w_i S'_jk with w_i = P_i r^2
//   (so rows <= j and columns <= j of A stay as they are); column j's owners
//   scale it, C_ij = A_ij r (i > j).
// Afterwards sA holds C below the diagonal and the last pivots A_ii on it, and
// sX holds X_ic = -S_ic r_i (c < i), r_i (c = i), zero above.
__device__ __forceinline__ void diag16(double *sA, double *sX, double *dC, double *dS, const int o,
                                       const int l, int &bad) {
    const int i = l >> 2, q = l & 3;
    double a[4], s[4], e[4], ri = 0.0;  // e: the identity's entries, ri: r of this lane's row
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        a[v] = sA[(o + i) * FP + o + 4 * v + q];
        s[v] = 0.0;
        e[v] = 4 * v + q == i ? 1.0 : 0.0;
    }
    double rn = rsqrt_nr(a[0]);  // every lane's own entry; lane 4 j + j % 4 holds the pivot's
#pragma unroll
    for (int j = 0; j < DB; ++j) {
        const int jv = j >> 2, qj = j & 3, pl = 4 * j + qj;
        double r = readlane_d(rn, pl);
        const double piv = readlane_d(a[jv], pl);
        if (!(piv > 0.0) || !isfinite(piv)) {
            bad = 1;
            r = rsqrt_nr(1.0);
        }
        // j as an opaque per-column value: the lane masks are then formed here
        // instead of all being hoisted ahead of the loop (which spills them)
        int jo;
        asm volatile("v_mov_b32 %0, %1" : "=v"(jo) : "i"(j));
        ri = i == jo ? r : ri;
        // lanes that publish nothing write their own spare slot, so there is no branch
        dC[q == qj ? (i & 3) * 4 + (i >> 2) : DB + l] = i > jo ? a[jv] : 0.0;
        {   // row j: S_jc is zero for c > j (those entries are never updated), so
            // S'_j = S_j - e_j
            double2 *ds = reinterpret_cast<double2 *>(i == jo ? dS + 4 * q : dS + DB + 4 * l);
            ds[0] = double2{s[0] - e[0], s[1] - e[1]};
            ds[1] = double2{s[2] - e[2], s[3] - e[3]};
        }
        lds_order();
        const double pr = dC[(i & 3) * 4 + (i >> 2)];
        const double2 c0 = reinterpret_cast<const double2 *>(dC + 4 * q)[0];
        const double2 c1 = reinterpret_cast<const double2 *>(dC + 4 * q)[1];
        const double2 x0 = reinterpret_cast<const double2 *>(dS + 4 * q)[0];
        const double2 x1 = reinterpret_cast<const double2 *>(dS + 4 * q)[1];
        lds_order();
        const double cv[4] = {c0.x, c0.y, c1.x, c1.y}, xv[4] = {x0.x, x0.y, x1.x, x1.y};
        const double w = pr * r * r;
        if (j + 1 < DB) {  // the next pivot's entry first, so its 1 / sqrt overlaps the rest
            const int nv = (j + 1) >> 2;
            a[nv] = fma(-w, cv[nv], a[nv]);
            rn = rsqrt_nr(a[nv]);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            if (j + 1 >= DB || v != ((j + 1) >> 2)) a[v] = fma(-w, cv[v], a[v]);
            s[v] = fma(-w, xv[v], s[v]);
        }
        if (q == qj) a[jv] = i > jo ? a[jv] * r : a[jv];
    }
    lds_order();
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int c = 4 * v + q;
        sA[(o + i) * FP + o + c] = a[v];
        sX[(o + i) * FP + o + c] = c < i ? -s[v] * ri : (c == i ? ri : 0.0);
    }
}

// One 64 x 64 diagonal block at (off, off): its Cholesky factor and the
// inverse of that factor, one workgroup, blocked by 16.  For the diagonal
// blocks p = 0..3 in turn (sA holds A, then C; sX the block sums S, then X):
//   (a) one wave factors and inverts the diagonal block (diag16);
//   (b) C_ip = A_ip X_pp^T (i > p) and X_pc = -X_pp S_pc (c < p);
//   (c) A_ik -= C_ip C_kp^T (p < k <= i) and S_ic += C_ip X_pc (i > p, c <= p);
// (b) and (c) are 16 x 16 x 16 products on the fp64 matrix cores, spread over
// the four waves, with a barrier before each phase.  In (c), wave 0 updates
// the next diagonal block first and factors it at once (its (a)), while waves
// 1..3 finish the other trailing blocks, which that block does not read.  This
// is the block form of
// the same recursion (C X = I by block forward substitution, S_pc the sum over
// m < p of C_pm X_mc).  The block goes in and out through LDS, so the global
// accesses are coalesced.
__device__ __forceinline__ void base_block(const double *G, double *X, int64_t dp, int64_t off, int &bad) {
    __shared__ double sA[FT * FP];
    __shared__ double sX[FT * FP];
    __shared__ __align__(16) double dC[DB + 64];      // the column, then one spare slot per lane
    __shared__ __align__(16) double dS[DB + 4 * 64];  // the pending row, then four spare slots per lane
    const int t = threadIdx.x, w = t >> 6, l = t & 63;
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int i = idx >> 6, k = idx & 63;
        sA[i * FP + k] = G[(off + i) * dp + off + k];
        sX[i * FP + k] = 0.0;
    }
    __syncthreads();
    if (w == 0) diag16(sA, sX, dC, dS, 0, l, bad);
    for (int p = 0; p < FT / DB; ++p) {
        const int o = DB * p;
        __syncthreads();
        // (b): 3 products, one per wave 1..3: C_ip for i = p+1..3, then X_pc for c = 0..p-1
        if (w > 0) {
            const int e = w - 1, nc = 3 - p;
            doublex4 acc{0.0, 0.0, 0.0, 0.0};
            if (e < nc) {
                const int i = p + 1 + e;
                mm16(acc, &sA[DB * i * FP + o], FP, &sX[o * FP + o], 1, FP, 1.0, l);
                st16(&sA[DB * i * FP + o], l, acc);
            } else {
                const int c = e - nc;
                mm16(acc, &sX[o * FP + o], FP, &sX[o * FP + DB * c], FP, 1, -1.0, l);
                st16(&sX[o * FP + DB * c], l, acc);
            }
        }
        __syncthreads();
        // (c): wave 0 updates the next diagonal block and factors it at once, while
        // waves 1..3 take the other trailing blocks round-robin
        if (w == 0) {
            if (p + 1 < FT / DB) {
                const int i = p + 1;
                doublex4 acc = ld16(&sA[DB * i * FP + DB * i], l);
                mm16(acc, &sA[DB * i * FP + o], FP, &sA[DB * i * FP + o], 1, FP, -1.0, l);
                st16(&sA[DB * i * FP + DB * i], l, acc);
                lds_order();
                diag16(sA, sX, dC, dS, DB * i, l, bad);
            }
        } else {
            int n = 0;
            for (int i = p + 1; i < FT / DB; ++i)
                for (int k = p + 1; k <= i; ++k) {
                    if (i == p + 1 && k == p + 1) continue;
                    if (n++ % 3 == w - 1) {
                        doublex4 acc = ld16(&sA[DB * i * FP + DB * k], l);
                        mm16(acc, &sA[DB * i * FP + o], FP, &sA[DB * k * FP + o], 1, FP, -1.0, l);
                        st16(&sA[DB * i * FP + DB * k], l, acc);
                    }
                }
            for (int i = p + 1; i < FT / DB; ++i)
                for (int c = 0; c <= p; ++c)
                    if (n++ % 3 == w - 1) {
                        doublex4 acc = ld16(&sX[DB * i * FP + DB * c], l);
                        mm16(acc, &sA[DB * i * FP + o], FP, &sX[o * FP + DB * c], FP, 1, 1.0, l);
                        st16(&sX[DB * i * FP + DB * c], l, acc);
                    }
        }
    }
    __syncthreads();
    for (int idx = t; idx < FT * FT; idx += 256) {
        const int i = idx >> 6, k = idx & 63;
        X[(off + i) * dp + off + k] = k <= i ? sX[i * FP + k] : 0.0;
    }
}

__global__ __launch_bounds__(256) void base_kernel(const double *__restrict__ G, double *X, int64_t dp,
                                                   int64_t off, int32_t *dev_status) {
    int bad = 0;
    base_block(G, X, dp, off, bad);
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
    int xcd;  // a 1-D grid whose workgroup x takes the output rows ib = x (mod 8) (mb % 8 = 0)
};

// The output tile (ib, jb) of TM x TM of one product, by one workgroup of 256
// threads: each wave takes a TM/2 x TM/2 quarter as (TM/32)^2 blocks of 16 x 16
// on the matrix cores.  Every output entry sums its k in the same order and in
// the same groups of four whatever TM is, so the tile size does not change the
// result; the skipped k blocks hold exact zeros.
template <int TM, int GK = 32>
__device__ __forceinline__ void dgemm_tile(const DGemm &g, const int ib, const int jb) {
    constexpr int GS = GK + 1;  // LDS row stride (doubles)
    constexpr int WT = TM / 2, NB = WT / 16;
    constexpr int LPT = TM * GK / 256;  // doubles of A (and of B) each thread moves per k chunk
    constexpr int TPR = GK / LPT;       // threads per row of A (and of B by row)
    constexpr int TPK = TM / LPT;       // threads per k row of B (bnn = 1)
    int klo = 0, khi = g.K;
    if (g.kmode == 1) khi = min(g.K, TM * (ib + 1));
    if (g.kmode == 2) khi = min(g.K, TM * (jb + 1));
    if (g.kmode == 3) klo = TM * jb;
    __shared__ double As[TM * GS];
    __shared__ double Bs[TM * GS];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int qr = w >> 1, qc = w & 1;
    doublex4 acc[NB][NB];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = doublex4{0.0, 0.0, 0.0, 0.0};
    // Each thread moves LPT consecutive doubles of A and of B per k chunk: A and
    // (bnn = 0) B by row (row t / TPR, k offset LPT (t % TPR)); B (bnn = 1) by k
    // row (t / TPK, columns LPT (t % TPK) ..).  The next chunk is read into
    // registers while the current one is multiplied.
    const int row = t / TPR, kk = (t % TPR) * LPT;
    const int kr = t / TPK, jj = (t % TPK) * LPT;
    const double *Asrc = g.A + ((int64_t)TM * ib + row) * g.lda + kk;
    const double *Bsrc = g.bnn ? g.B + (int64_t)kr * g.ldb + (int64_t)TM * jb + jj
                               : g.B + ((int64_t)TM * jb + row) * g.ldb + kk;
    const int64_t bstep = g.bnn ? (int64_t)g.ldb : 1;  // B address advance per unit of k
    // the old values of an updated tile, read now so their latency overlaps the loop
    double cold[NB][NB][4];
    if (g.beta != 0.0) {
#pragma unroll
        for (int a = 0; a < NB; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t row = (int64_t)TM * ib + WT * qr + 16 * a + (lane >> 4) + 4 * v;
                    const int64_t col = (int64_t)TM * jb + WT * qc + 16 * b + (lane & 15);
                    cold[a][b][v] = g.C[row * g.ldc + col];
                }
    }
    double ra[LPT], rb[LPT];
    if (klo < khi) {
#pragma unroll
        for (int q = 0; q < LPT; ++q) {
            ra[q] = Asrc[klo + q];
            rb[q] = Bsrc[klo * bstep + q];
        }
    }
    for (int k0 = klo; k0 < khi; k0 += GK) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < LPT; ++q) As[row * GS + kk + q] = ra[q];
        if (!g.bnn) {
#pragma unroll
            for (int q = 0; q < LPT; ++q) Bs[row * GS + kk + q] = rb[q];
        } else {
#pragma unroll
            for (int q = 0; q < LPT; ++q) Bs[(jj + q) * GS + kr] = rb[q];
        }
        __syncthreads();
        if (k0 + GK < khi) {
            const int kn = k0 + GK;
#pragma unroll
            for (int q = 0; q < LPT; ++q) {
                ra[q] = Asrc[kn + q];
                rb[q] = Bsrc[kn * bstep + q];
            }
        }
        // lane l supplies A[l % 16][k] and B[k][l % 16] with k = 4 s + l / 16
#pragma unroll
        for (int s = 0; s < GK / 4; ++s) {
            double av[NB], bv[NB];
#pragma unroll
            for (int a = 0; a < NB; ++a) av[a] = As[(WT * qr + 16 * a + (lane & 15)) * GS + 4 * s + (lane >> 4)];
#pragma unroll
            for (int b = 0; b < NB; ++b) bv[b] = Bs[(WT * qc + 16 * b + (lane & 15)) * GS + 4 * s + (lane >> 4)];
#pragma unroll
            for (int a = 0; a < NB; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
        }
    }
    // register v of lane l holds D[l / 16 + 4 v][l % 16] of each 16 x 16 block
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = (int64_t)TM * ib + WT * qr + 16 * a + (lane >> 4) + 4 * v;
                const int64_t col = (int64_t)TM * jb + WT * qc + 16 * b + (lane & 15);
                const double r = g.alpha * acc[a][b][v];
                g.C[row * g.ldc + col] = g.beta != 0.0 ? fma(g.beta, cold[a][b][v], r) : r;
            }
}

template <int TM>
__global__ __launch_bounds__(256) void dgemm_kernel(DGemm g) {
    int ib, jb;
    if (g.lower) {
        const int64_t x = blockIdx.x;
        int64_t a = (int64_t)((sqrt(8.0 * (double)x + 1.0) - 1.0) * 0.5);
        while (a * (a + 1) / 2 > x) --a;
        while ((a + 1) * (a + 2) / 2 <= x) ++a;
        ib = (int)a;
        jb = (int)(x - a * (a + 1) / 2);
    } else if (g.xcd) {
        // linear workgroup ids reach the 8 XCDs round-robin: XCD x takes the rows
        // ib = x (mod 8), a whole row at a time, so a row's A panel is read into one L2
        const int nb = g.N / TM, x = blockIdx.x & 7, k = blockIdx.x >> 3;
        ib = x + 8 * (k / nb);
        jb = k % nb;
    } else {
        ib = blockIdx.y;
        jb = blockIdx.x;
    }
    dgemm_tile<TM>(g, ib, jb);
}

// A whole 128 x 128 recursion node at (off, off) in one workgroup: the two
// diagonal blocks and the four one-tile products between them, in the order
// and with the arithmetic of the separate launches (so the result is the
// same), without five launches in between.  The workgroup's global writes are
// visible to its own later reads after each barrier.
__global__ __launch_bounds__(256) void node128_kernel(double *G, double *C, double *X, double *T,
                                                      int64_t dp, int64_t off, int32_t *dev_status) {
    auto at = [dp](double *p, int64_t r, int64_t c) { return p + r * dp + c; };
    const int64_t o2 = off + FT;
    int bad = 0;
    base_block(G, X, dp, off, bad);
    __syncthreads();
    // C21 = G21 X11^T
    dgemm_tile<FT, FT>(DGemm{at(G, o2, off), dp, at(X, off, off), dp, at(C, o2, off), dp, FT, FT, FT, 0, 2, 0, 1.0, 0.0, 0},
               0, 0);
    __syncthreads();
    // G22 -= C21 C21^T
    dgemm_tile<FT, FT>(DGemm{at(C, o2, off), dp, at(C, o2, off), dp, at(G, o2, o2), dp, FT, FT, FT, 0, 0, 1, -1.0, 1.0, 0},
               0, 0);
    __syncthreads();
    base_block(G, X, dp, o2, bad);
    __syncthreads();
    // T = C21 X11, X21 = -X22 T
    dgemm_tile<FT, FT>(DGemm{at(C, o2, off), dp, at(X, off, off), dp, at(T, o2, off), dp, FT, FT, FT, 1, 3, 0, 1.0, 0.0, 0},
               0, 0);
    __syncthreads();
    dgemm_tile<FT, FT>(DGemm{at(X, o2, o2), dp, at(T, o2, off), dp, at(X, o2, off), dp, FT, FT, FT, 1, 1, 0, -1.0, 0.0, 0},
               0, 0);
    if (bad && dev_status) atomicOr(dev_status, BAKRON_DEV_NOT_PD);
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

// Nodes at least this wide run T = C21 X11 on a side stream, beside the
// recursion into G22 (T needs only C21 and X11; the recursion is latency-bound
// and leaves most of the GPU idle), and join it before X21 = -X22 T.
constexpr int64_t SIDE_T_MIN = 1024;

// Per device: the side stream and a pool of fork / join events, used under
// one lock for the whole enqueue of a factor call.
struct FactorSide {
    hipStream_t side = nullptr;
    std::vector<hipEvent_t> ev;
};
std::mutex g_fside_mu;
std::map<int, FactorSide> g_fside;

struct Factor {
    FBufs f;
    int64_t dp;
    int32_t *dev_status;
    hipStream_t stream;
    hipStream_t side;  // nullptr: every step on stream
    FactorSide *fs;
    mutable int nev;   // events of fs taken so far
};

// XCD-aware tile order for wide outputs (measured: 2.6 % faster at d = 14336,
// where the top products are 112 tiles wide; no gain at 32 tiles wide).
template <int TM>
void launch_gemm(DGemm g, const int M, const int N, const hipStream_t stream) {
    const int mb = M / TM, nb = N / TM;
    if (g.lower) {
        hipLaunchKernelGGL(dgemm_kernel<TM>, dim3((unsigned)(mb * (mb + 1) / 2)), dim3(256), 0, stream, g);
    } else if (mb % 8 == 0 && nb >= 64) {
        g.xcd = 1;
        hipLaunchKernelGGL(dgemm_kernel<TM>, dim3((unsigned)(mb * nb)), dim3(256), 0, stream, g);
    } else {
        hipLaunchKernelGGL(dgemm_kernel<TM>, dim3(nb, mb), dim3(256), 0, stream, g);
    }
}

// The tile size: 64 if that still gives at least one workgroup per compute
// unit, else 32 (an fp64 tile runs at one compute unit's matrix rate, so small
// products need small tiles).  Tiles stay at most 64 wide: the k range a
// triangular operand skips is cut at the tile's own rows or columns, and only
// the diagonal 64 x 64 blocks of C and X have their upper part written (as
// zeros), so a wider tile would read blocks above the diagonal that are never
// written.
int gemm_tile(const int M, const int N, const int lower) {
    const int64_t mb = M / FT, nb = N / FT;
    return (lower ? mb * (mb + 1) / 2 : mb * nb) >= 256 ? FT : 32;
}

int32_t gemm(const Factor &fc, const double *A, const double *B, double *Cout, int M, int N, int K,
             int bnn, int kmode, int lower, double alpha, double beta, hipStream_t stream = nullptr) {
    const DGemm g{A, fc.dp, B, fc.dp, Cout, fc.dp, M, N, K, bnn, kmode, lower, alpha, beta, 0};
    if (!stream) stream = fc.stream;
    if (gemm_tile(M, N, lower) == FT) launch_gemm<FT>(g, M, N, stream);
    else launch_gemm<32>(g, M, N, stream);
    BK_LAUNCH_CHECK("dgemm_kernel");
    return BAKRON_OK;
}

int32_t take_event(const Factor &fc, hipEvent_t *e) {
    if (fc.nev == (int)fc.fs->ev.size()) {
        hipEvent_t n;
        BK_HIP_CHECK(hipEventCreateWithFlags(&n, hipEventDisableTiming));
        fc.fs->ev.push_back(n);
    }
    *e = fc.fs->ev[fc.nev++];
    return BAKRON_OK;
}

// factor and invert the diagonal block [off, off + n) of G into C and X
int32_t recurse(const Factor &fc, int64_t off, int64_t n) {
    const int64_t dp = fc.dp;
    if (n == FT) {
        hipLaunchKernelGGL(base_kernel, dim3(1), dim3(256), 0, fc.stream, fc.f.G, fc.f.X, dp, off,
                           fc.dev_status);
        BK_LAUNCH_CHECK("base_kernel");
        return BAKRON_OK;
    }
    if (n == 2 * FT) {
        hipLaunchKernelGGL(node128_kernel, dim3(1), dim3(256), 0, fc.stream, fc.f.G, fc.f.C, fc.f.X,
                           fc.f.T, dp, off, fc.dev_status);
        BK_LAUNCH_CHECK("node128_kernel");
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
    // T = C21 X11 (X11 lower: rows k >= the output column block): on the side
    // stream for wide nodes (its region of T is this node's alone)
    const bool side = fc.side && n >= SIDE_T_MIN;
    hipEvent_t fork = nullptr, join = nullptr;
    if (side) {
        st = take_event(fc, &fork);
        if (st == BAKRON_OK) st = take_event(fc, &join);
        if (st != BAKRON_OK) return st;
        BK_HIP_CHECK(hipEventRecord(fork, fc.stream));
        BK_HIP_CHECK(hipStreamWaitEvent(fc.side, fork, 0));
    }
    st = gemm(fc, at(C, off + n1, off), at(X, off, off), at(T, off + n1, off), (int)n2, (int)n1,
              (int)n1, 1, 3, 0, 1.0, 0.0, side ? fc.side : fc.stream);
    if (st != BAKRON_OK) return st;
    if (side) BK_HIP_CHECK(hipEventRecord(join, fc.side));
    // G22 -= C21 C21^T, lower tiles
    st = gemm(fc, at(C, off + n1, off), at(C, off + n1, off), at(G, off + n1, off + n1), (int)n2,
              (int)n2, (int)n1, 0, 0, 1, -1.0, 1.0);
    if (st != BAKRON_OK) return st;
    st = recurse(fc, off + n1, n2);
    if (st != BAKRON_OK) return st;
    // X21 = -X22 T (X22 lower)
    if (side) BK_HIP_CHECK(hipStreamWaitEvent(fc.stream, join, 0));
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
    fc.side = nullptr;
    fc.fs = nullptr;
    fc.nev = 0;
    fcarve(ws, fc.dp, &fc.f);
    // The side stream is shared by the device's factor calls, so a call being
    // captured into a graph keeps every step on its own stream.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    BK_HIP_CHECK(hipStreamIsCapturing(stream, &cap));
    int dev = 0;
    BK_HIP_CHECK(hipGetDevice(&dev));
    std::unique_lock<std::mutex> lock(g_fside_mu, std::defer_lock);
    if (cap == hipStreamCaptureStatusNone && fc.dp >= 2 * SIDE_T_MIN) {
        lock.lock();
        FactorSide &fs = g_fside[dev];
        if (!fs.side) BK_HIP_CHECK(hipStreamCreateWithFlags(&fs.side, hipStreamNonBlocking));
        fc.side = fs.side;
        fc.fs = &fs;
    }
    hipLaunchKernelGGL(load_reversed_kernel, dim3(2048), dim3(256), 0, stream, H, d, fc.f.G, fc.dp);
    BK_LAUNCH_CHECK("load_reversed_kernel");
    st = recurse(fc, 0, fc.dp);
    if (st != BAKRON_OK) return st;
    const unsigned tl = (unsigned)((d + FT - 1) / FT);
    hipLaunchKernelGGL(write_l_kernel, dim3(tl, tl), dim3(256), 0, stream, fc.f.X, fc.dp, d, L);
    BK_LAUNCH_CHECK("write_l_kernel");
    return BAKRON_OK;
}
