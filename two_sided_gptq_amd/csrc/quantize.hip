// quantize.hip -- bakron_quantize, the solver's hot path, for gfx950.
//
// Method: BaKron / FastKron (arXiv 2608.06291), as described on the
// pith.science review page ("What carries the argument": Proposition 3.1,
// anti-diagonal independence, band updates batched into two matrix products;
// "Core claim": Theorem 3.2, O(m+n) sequential steps and O(mn(m+n)) work) and
// the mlsanity.com index page (abstract).
//
// Pipeline for one call, all enqueued on the caller's stream:
//   1. qparams    per-row scale / zero point from the original W
//   2. relayout   W -> padded fp32 working copy Wp (mp x np, multiples of 64);
//                 LA, LB -> padded lower-triangular copies (identity padding)
//   3. schedule   in-order walk of the recursion over 64 x 64 TILE
//                 anti-diagonals K = I + J (tiles on one tile anti-diagonal are
//                 independent, for the same reason single entries on one
//                 anti-diagonal are):
//                   leaf(K)        one workgroup per tile, the whole in-tile
//                                  problem solved in LDS, 127 diagonal steps
//                   band(K, L, H)  postponed update from tile diagonals
//                                  S = [K, K+H) to R = [K+H, K+L) as two
//                                  staircase fp32-MFMA GEMMs
//   4. finalise   sum of e^2 in a fixed order
#include <algorithm>
#include <climits>
#include <cstddef>
#include <map>
#include <mutex>
#include <vector>

#include "common.hpp"

namespace bakron {
namespace {

constexpr int TB = 64;  // tile edge (leaf tile and band-GEMM output tile)
constexpr int LP = 80;  // LDS row stride in floats for the leaf tiles
constexpr int GP = 68;  // LDS row stride in floats for the GEMM operand tiles
constexpr int NPART = 1024;  // partial sums of the e^2 reduction

typedef float floatx16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ qparams
// Per-row scale shrink by MSE search (review page, free parameters: the
// per-row scale shrinks by up to a factor 2, chosen by an MSE search).  The
// candidates scale the row's range (max |w|, or min w and max w) by
// p_k = (MSE_GRID - k) / MSE_GRID, k = 0 .. MSE_MAXK, and take the plain
// parameters of the shrunk range; a candidate's error is the row's sum of
// (w - v)^2, v the base quantizer's clamped value of w on that grid; the first
// candidate with the least error wins.  Parameters and v in fp32 (no fused
// operations), squared errors summed in fp64: per thread over j = t (mod 256),
// then a fixed butterfly in each wave and the four waves in order.  k = 0 is
// the plain quantizer.  All 256 threads call it; returns (s, z) to all.
constexpr int MSE_GRID = 100, MSE_MAXK = 50;

__device__ void mse_search(const float *row, int64_t n, int kind, int bits, float amax, float lo,
                           float hi, float &s_out, float &z_out) {
#pragma clang fp contract(off)
    __shared__ double red[4];
    __shared__ float best_s, best_z;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float qmin = kind == BAKRON_Q_SYM ? -(float)(1 << (bits - 1)) : 0.0f;
    const float qmax = kind == BAKRON_Q_SYM ? (float)((1 << (bits - 1)) - 1) : (float)((1 << bits) - 1);
    double best = INFINITY;  // meaningful in thread 0
    for (int k = 0; k <= MSE_MAXK; ++k) {
        const float p = (float)(MSE_GRID - k) / (float)MSE_GRID;
        float s, z = 0.0f;
        if (kind == BAKRON_Q_SYM) {
            const float a = amax * p;
            s = a / qmax;
            if (s == 0.0f) s = 1.0f;
        } else {
            const float lo_p = lo * p, hi_p = hi * p;
            const float range = hi_p - lo_p;
            s = range / qmax;
            if (s == 0.0f) s = 1.0f;
            else z = fminf(fmaxf(rintf(-lo_p / s), 0.0f), qmax);
        }
        double acc = 0.0;
        for (int64_t j = t; j < n; j += 256) {
            const float x = row[j];
            const float c = fminf(fmaxf(rintf(x / s) + z, qmin), qmax);
            const float v = s * (c - z);
            const double d = (double)x - (double)v;
            const double d2 = d * d;
            acc = acc + d2;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const double o = __shfl_xor(acc, off);
            acc = acc + o;
        }
        if (lane == 0) red[w] = acc;
        __syncthreads();
        if (t == 0) {
            const double err = ((red[0] + red[1]) + red[2]) + red[3];
            if (err < best) {
                best = err;
                best_s = s;
                best_z = z;
            }
        }
        __syncthreads();
    }
    s_out = best_s;
    z_out = best_z;
}

// One workgroup per padded row (row0 + block).  Rows >= m get s = 1, z = 0 (the padding is
// all zeros, so every padded entry rounds to its zero point exactly).  With
// mse (symmetric and asymmetric kinds) the scale shrink comes from mse_search.
// With Wp, the workgroup also writes its row of the padded working copy
// (row stride np, zeros past n; padded rows all zero) as it reads the row.
__global__ __launch_bounds__(256) void qparams_kernel(
    const float *__restrict__ W, int64_t m, int64_t n, int kind, int bits,
    float *__restrict__ scales, float *__restrict__ zeros, float *__restrict__ sc_pad,
    float *__restrict__ zp_pad, int32_t *dev_status, int mse, int vec, float *__restrict__ Wp,
    int64_t np, int64_t row0) {
    __shared__ float s_amax[4], s_lo[4], s_hi[4];
    __shared__ int s_bad[4];
    const int64_t i = row0 + blockIdx.x;
    const int t = threadIdx.x;
    float s = 1.0f, z = 0.0f;
    float *wrow = Wp ? Wp + i * np : nullptr;
    if (wrow) {  // the padding: columns n .. np-1, or the whole of a padded row
        const int64_t from = i < m ? n : 0;
        if ((from & 3) == 0) {
            for (int64_t j = from + 4 * t; j < np; j += 4 * 256)
                *reinterpret_cast<float4 *>(wrow + j) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            for (int64_t j = from + t; j < np; j += 256) wrow[j] = 0.0f;
        }
    }
    if (i < m) {
        float amax = 0.0f, lo = INFINITY, hi = -INFINITY;
        int bad = 0;
        const float *row = W + i * n;
        auto take = [&](float w) {
            bad |= !isfinite(w);
            amax = fmaxf(amax, fabsf(w));
            lo = fminf(lo, w);
            hi = fmaxf(hi, w);
        };
        if (vec) {  // four float4 loads in flight per thread
            const float4 *r4 = reinterpret_cast<const float4 *>(row);
            float4 *w4 = reinterpret_cast<float4 *>(wrow);
            const int64_t n4 = n / 4;
            int64_t j = t;
            for (; j + 3 * 256 < n4; j += 4 * 256) {
                const float4 a = r4[j], b = r4[j + 256], c = r4[j + 512], d = r4[j + 768];
                if (w4) {
                    w4[j] = a;
                    w4[j + 256] = b;
                    w4[j + 512] = c;
                    w4[j + 768] = d;
                }
                take(a.x); take(a.y); take(a.z); take(a.w);
                take(b.x); take(b.y); take(b.z); take(b.w);
                take(c.x); take(c.y); take(c.z); take(c.w);
                take(d.x); take(d.y); take(d.z); take(d.w);
            }
            for (; j < n4; j += 256) {
                const float4 a = r4[j];
                if (w4) w4[j] = a;
                take(a.x); take(a.y); take(a.z); take(a.w);
            }
        } else {
            for (int64_t j = t; j < n; j += 256) {
                const float w = row[j];
                if (wrow) wrow[j] = w;
                take(w);
            }
        }
        // max, min and or are exact in any order: a butterfly in each wave,
        // then the four waves' values
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            amax = fmaxf(amax, __shfl_xor(amax, off));
            lo = fminf(lo, __shfl_xor(lo, off));
            hi = fmaxf(hi, __shfl_xor(hi, off));
            bad |= __shfl_xor(bad, off);
        }
        const int w = t >> 6;
        if ((t & 63) == 0) {
            s_amax[w] = amax;
            s_lo[w] = lo;
            s_hi[w] = hi;
            s_bad[w] = bad;
        }
        __syncthreads();
        if (t == 0) {
            s_amax[0] = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
            s_lo[0] = fminf(fminf(s_lo[0], s_lo[1]), fminf(s_lo[2], s_lo[3]));
            s_hi[0] = fmaxf(fmaxf(s_hi[0], s_hi[1]), fmaxf(s_hi[2], s_hi[3]));
            s_bad[0] = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];
        }
        __syncthreads();
        if (kind == BAKRON_Q_SYM) {
            s = s_amax[0] / (float)((1 << (bits - 1)) - 1);  // IEEE fp32 division
            if (s == 0.0f) s = 1.0f;
        } else if (kind == BAKRON_Q_ASYM) {
            const float qmax = (float)((1 << bits) - 1);
            const float range = s_hi[0] - s_lo[0];
            s = range / qmax;
            if (s == 0.0f) {
                s = 1.0f;
            } else {
                z = fminf(fmaxf(rintf(-s_lo[0] / s), 0.0f), qmax);
            }
        }
        if (mse && kind != BAKRON_Q_UNIT && !s_bad[0])
            mse_search(row, n, kind, bits, s_amax[0], s_lo[0], s_hi[0], s, z);
        if (t == 0) {
            scales[i] = s;
            if (zeros) zeros[i] = z;
            if (s_bad[0] && dev_status) atomicOr(dev_status, BAKRON_DEV_NONFINITE);
        }
    }
    if (t == 0) {
        sc_pad[i] = s;
        zp_pad[i] = z;
    }
}

// ----------------------------------------------------------------- relayout
// dst (prow x pcol, pcol % 4 == 0) from src (rows x cols).  tri = 0: plain
// copy with zero padding.  tri = 1: lower triangle of a square factor, upper
// part zero, padded diagonal one (so padded entries never divide by zero and
// never couple to real ones).  tri = 2: as 1, without the 64 x 64 blocks
// above the diagonal blocks, which the solve's kernels never read.  Rows
// row0 .. row1-1 of dst; each thread writes one float4.
__global__ __launch_bounds__(256) void relayout_kernel(
    const float *__restrict__ src, int64_t rows, int64_t cols, float *__restrict__ dst,
    int64_t prow, int64_t pcol, int tri, int vec_ok, int64_t row0, int64_t row1) {
    const int64_t q4 = pcol / 4;
    const int64_t total = min(row1, prow) * q4;
    for (int64_t idx = row0 * q4 + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = idx / q4;
        const int64_t c0 = (idx - r * q4) * 4;
        if (tri == 2 && c0 / TB > r / TB) continue;
        float v[4];
        const bool read = r < rows && !(tri && c0 > r);  // a factor's strictly upper part is not read
        if (read && vec_ok && c0 + 3 < cols) {
            const float4 x = *reinterpret_cast<const float4 *>(src + r * cols + c0);
            v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                v[k] = (read && c0 + k < cols) ? src[r * cols + c0 + k] : 0.0f;
        }
        if (tri) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t c = c0 + k;
                if (r < rows && c < cols) {
                    if (c > r) v[k] = 0.0f;
                } else {
                    v[k] = (c == r) ? 1.0f : 0.0f;
                }
            }
        }
        *reinterpret_cast<float4 *>(dst + r * pcol + c0) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// The leaf's per-column LA band table and per-row 1 / LB_rr, once per solve
// from the padded factors (the leaf used to build them from its LDS tiles
// behind a second barrier).  Entry x < np: column x of the grid, in its
// diagonal block J = x / TB at c = x % TB: LA[x][x - j] for j <= c (j < 8),
// zero for j > c, and 1 / LA_xx; entry x < mp: 1 / LB_xx.  Columns a0 .. a1-1
// and rows b0 .. b1-1.  Workgroup 0 also clears the nctr tile counters of the
// deferred band products (nctr = 0: none).
__global__ __launch_bounds__(256) void tables_kernel(const float *__restrict__ LAp,
                                                     const float *__restrict__ LBp, int64_t np,
                                                     int64_t mp, float4 *tabA, float *tabI, float *ilb,
                                                     int *ctr, int nctr, int64_t a0, int64_t a1,
                                                     int64_t b0, int64_t b1) {
    if (blockIdx.x == 0)
        for (int k = threadIdx.x; k < nctr; k += 256) ctr[k] = 0;
    const int64_t lo = min(a0, b0), hi = max(min(a1, np), min(b1, mp));
    for (int64_t x = lo + blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < hi;
         x += (int64_t)gridDim.x * blockDim.x) {
        if (x >= a0 && x < a1 && x < np) {
            const int c = (int)(x % TB);
            float band[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) band[j] = c >= j ? LAp[x * np + x - j] : 0.0f;
            tabA[2 * x] = make_float4(band[0], band[1], band[2], band[3]);
            tabA[2 * x + 1] = make_float4(band[4], band[5], band[6], band[7]);
            tabI[x] = band[0] != 0.0f ? 1.0f / band[0] : 0.0f;
        }
        if (x >= b0 && x < b1 && x < mp) ilb[x] = 1.0f / LBp[x * mp + x];
    }
}

// --------------------------------------------------------------------- leaf
struct LeafArgs {
    const float *Wp;  // mp x np working weights (all outside contributions applied)
    float *Ebuf;      // order 1: E (mp x np); order 2: E^T (np x mp)
    const float *LAp, *LBp;
    const float *sc, *zp;
    int64_t mp, np;
    int M, N, order;
    int qmin, qmax;
    int8_t *codes;
    float *V, *E;
    int64_t m, n;     // bounds of the outputs (rows, columns of the solved block)
    int32_t *dev_status;
    float *Cd, *Cr;   // contributions of the previous tile diagonal: from the tile above / to the left
    int out_vec;      // ldo % 4 == 0, codes 4-byte and V, E 16-byte aligned: outputs in groups of 4
    int64_t ldo;      // row stride of codes, V and E
    const float4 *tabA;  // column c of the grid: LA[c][c], LA[c][c-1 .. c-7] within its diagonal block
    const float *tabI;   // column c: 1 / LA_cc (0 where LA_cc is 0)
    const float *ilb;    // row r: 1 / LB_rr
};


__device__ inline float dot4(const float4 a, const float4 b, float s) {
    s = fmaf(a.x, b.x, s);
    s = fmaf(a.y, b.y, s);
    s = fmaf(a.z, b.z, s);
    s = fmaf(a.w, b.w, s);
    return s;
}

// The in-tile problem is the same two-sided rounding on a 64 x 64 block with
// the diagonal blocks LB[I,I], LA[J,J].  It is solved in the order-free form
// (each entry's value before rounding is W minus the contributions of every
// entry before it in the product order):
//   Z[r][c] = sum_{k <= c} E[r][k] LA[c][k]                  (row direction)
//   P[r][c] = W[r][c] - LB[r][r] sum_{k < c} E[r][k] LA[c][k]
//                     - sum_{k < r} LB[r][k] Z[k][c]         (column direction)
// Step d rounds the in-tile anti-diagonal r + c = d (127 steps).
//
// Wave 0 is the chain: lane r owns row r for the whole sweep (it is active at
// steps r .. r+63) and rounds entry (r, d - r) at step d.  The two dots are
// split at a boundary s0 that moves every LJ steps: terms produced before
// step s0 (the bulk) come precomputed by the helper waves, the rest
// (the last LJ..2LJ-1 terms of each dot) the chain adds itself:
//   row direction     its own last errors E[r][c-j], kept in registers;
//   column direction  Z[r-j][c], which lane r-j produced j steps ago.  Lane r
//                     keeps those in a delay line that is shifted down one
//                     lane per step with a whole-wave DPP shift, so the value
//                     just produced by the lane above arrives without LDS or
//                     a barrier.
// The chain and the helpers meet at a workgroup barrier once every LJ steps:
// during block t (steps LJ t .. LJ t + LJ - 1) the helpers compute the bulk
// of block t+1 from the E and Z values of steps < LJ t, which the previous
// barrier made visible, into the other half of a double buffer (the helper
// units are described at leaf_helpers).
constexpr int LJ = 4;                               // chain steps per block
constexpr int LWIN = 2 * LJ - 1;                    // most recent terms per dot
constexpr int NBLK = (2 * TB - 1 + LJ - 1) / LJ;    // blocks covering the sweep
constexpr int NSTEP = NBLK * LJ;                    // steps including the idle tail
constexpr int LEAF_THREADS = 768;                   // 12 waves, three per SIMD (wave w on SIMD w % 4)
constexpr int WSP = NSTEP + 4;                      // row stride of the skewed W copy
constexpr int CX = TB;                              // index of column 0 in the padded LA tables
constexpr int NCX = CX + NSTEP + 4;                 // padded LA table length (columns -64 .. 131)
static_assert(LWIN <= 7, "the LA band holds sub-diagonals 1..7");
static_assert(WSP % 4 == 0 && LJ == 4, "one float4 of W per block; 4-lane helper groups");
static_assert(NBLK % 2 == 0, "the chain alternates two operand buffers");

__shared__ __align__(16) float lf_Wk[TB * WSP];  // lf_Wk[r][d] = W[r][d - r] (row r skewed by r);
                                                 // after step d the slot holds that entry's code
__shared__ __align__(16) float lf_E[TB * LP];
__shared__ __align__(16) float lf_Z[TB * LP];    // lf_Z[c][k] = Z[k][c]
__shared__ __align__(16) float lf_B[TB * LP];    // LB[I,I]
__shared__ __align__(16) float lf_A[TB * LP];    // LA[J,J]
// The chain's per-step tables carry a larger alignment so that they are laid out
// before the big arrays, below 64 KB, where a load's constant part fits the
// instruction's offset field.
__shared__ __align__(32) float4 lf_Ab[NCX * 2];  // CX + c: LA[c][c], LA[c][c-1 .. c-7]; 0 off 0..63
__shared__ __align__(32) float lf_ila[NCX];      // CX + c: 1 / LA_cc; 0 off 0..63
__shared__ float4 lf_row[TB];                    // (s, 1/s, z, 1/LB_rr)
__shared__ __align__(32) float lf_bulk[2 * 2 * TB * LJ];  // [buffer][direction][row][step in block]
__shared__ float lf_sink[3 * TB];                // write targets of idle lanes
__shared__ __align__(16) float lf_P[2 * TB * GP]; // push operands: LA(J+1,J), then LB(I+1,I);
                                                  // a pulling leaf: the pushed V, skewed like W
static_assert(TB * WSP <= 2 * TB * GP, "the skewed V fits the push operands' area");

// the value lane l-1 holds, in lane l (lane 0 gets 0): a whole-wave shift
__device__ __forceinline__ float from_lane_above(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x138, 0xF, 0xF, true));
}


// wave 0; lane r = row r.  Every per-step LDS address is linear in the step d:
// W is stored skewed, the LA tables are padded over every column the lane
// passes, and idle lanes write to their own sink words.  The constant
// operands of block t+1 are loaded while block t runs.
struct ChainBlock {
    float4 w4;           // W[r][d - r] for the block's LJ steps
    float4 v4;           // pulling leaf: V[r][d - r] for the block's LJ steps
    float4 a[LJ][2];     // LA band of each step's column
    float ila[LJ];       // 1 / LA_cc of each step's column
};

template <bool PV>
__device__ __forceinline__ void chain_load(ChainBlock &cb, const float *wrow, const float4 *ab,
                                           const float *ib, int t) {
    cb.w4 = *reinterpret_cast<const float4 *>(wrow + LJ * t);
    if (PV) cb.v4 = *reinterpret_cast<const float4 *>(wrow - lf_Wk + lf_P + LJ * t);
#pragma unroll
    for (int p = 0; p < LJ; ++p) {
        const int d = LJ * t + p;
        cb.a[p][0] = ab[2 * d];
        cb.a[p][1] = ab[2 * d + 1];
        cb.ila[p] = ib[d];
    }
}

struct ChainState {
    float lbb[LWIN + 1];   // LB[r][r - j]
    float4 rc;             // (s, 1/s, z, 1/LB_rr)
    float qminf, qmaxf;
    float eh[LWIN], zl[LWIN];  // eh[j] = E[r][c-1-j], zl[j] = Z[r-1-j][c]
    float *wrow;           // the lane's row of the skewed W copy; its consumed slots take the codes
    int r, e_off, z_off;
};

// Block t: the bulk of its steps is read first (it is the only operand the
// helpers wrote during the previous block), then the next block's constant
// operands are requested, then the LJ steps run.  PV: the leaf pulls V, which
// starts each entry's row-direction sum.
template <bool ZP, bool PV>
__device__ __forceinline__ void chain_block(ChainState &st, const ChainBlock &cb, ChainBlock &next,
                                            const float *wrow, const float4 *ab, const float *ib,
                                            int t) {
    const int r = st.r;
    float bulk1[LJ], bulk2[LJ], code[LJ];
#pragma unroll
    for (int p = 0; p < LJ; ++p) {
        bulk1[p] = lf_bulk[(((t & 1) * 2 + 0) * TB + r) * LJ + p];
        bulk2[p] = lf_bulk[(((t & 1) * 2 + 1) * TB + r) * LJ + p];
    }
    chain_load<PV>(next, wrow, ab, ib, t + 1);
    const float wv[4] = {cb.w4.x, cb.w4.y, cb.w4.z, cb.w4.w};
    const float vv[4] = {cb.v4.x, cb.v4.y, cb.v4.z, cb.v4.w};
#pragma unroll
    for (int p = 0; p < LJ; ++p) {
        const int d = LJ * t + p;
        const float la[8] = {cb.a[p][0].x, cb.a[p][0].y, cb.a[p][0].z, cb.a[p][0].w,
                             cb.a[p][1].x, cb.a[p][1].y, cb.a[p][1].z, cb.a[p][1].w};
        // the bulk, then the recent terms j = LJ + p .. 2 (steps s0 .. d-2),
        // then the fresh j = 1
        float y = PV ? bulk1[p] + vv[p] : bulk1[p], s2 = bulk2[p];
#pragma unroll
        for (int j = LJ + p; j >= 2; --j) {
            y = fmaf(st.eh[j - 1], la[j], y);
            s2 = fmaf(st.lbb[j], st.zl[j - 1], s2);
        }
        y = fmaf(st.eh[0], la[1], y);
        s2 = fmaf(st.lbb[1], st.zl[0], s2);
        const float P = wv[p] - fmaf(st.lbb[0], y, s2);
        // code = clamp(rint(P / s) + z), value s (code - z)
        float qz, res;
        if (ZP) {
            qz = __builtin_amdgcn_fmed3f(rintf(P * st.rc.y) + st.rc.z, st.qminf, st.qmaxf);
            res = fmaf(-st.rc.x, qz - st.rc.z, P);
        } else {
            qz = __builtin_amdgcn_fmed3f(rintf(P * st.rc.y), st.qminf, st.qmaxf);
            res = fmaf(-st.rc.x, qz, P);
        }
        const bool act = (unsigned)(d - r) < (unsigned)TB;
        float e = res * (st.rc.w * cb.ila[p]);
        float z = fmaf(e, la[0], y);
        code[p] = qz;
        *(act ? lf_E + st.e_off + d : lf_sink + r) = e;
        *(act ? lf_Z + st.z_off + d * LP : lf_sink + TB + r) = z;
#pragma unroll
        for (int j = LWIN - 1; j >= 1; --j) {
            st.eh[j] = st.eh[j - 1];
            st.zl[j] = from_lane_above(st.zl[j - 1]);
        }
        st.eh[0] = e;
        st.zl[0] = from_lane_above(z);
    }
    // the block's W slots were read before the block started
    *reinterpret_cast<float4 *>(st.wrow + LJ * t) = make_float4(code[0], code[1], code[2], code[3]);
}

template <bool ZP, bool PV>
__device__ __forceinline__ void leaf_chain(const int r, const float qminf, const float qmaxf) {
    __builtin_assume(r >= 0 && r < TB);
    ChainState st;
    st.r = r;
    st.lbb[0] = lf_B[r * LP + r];
#pragma unroll
    for (int j = 1; j <= LWIN; ++j) st.lbb[j] = r >= j ? lf_B[r * LP + r - j] : 0.0f;
    st.rc = lf_row[r];
    st.qminf = qminf;
    st.qmaxf = qmaxf;
#pragma unroll
    for (int j = 0; j < LWIN; ++j) st.eh[j] = st.zl[j] = 0.0f;
    st.e_off = r * (LP - 1);   // E[r][d - r]
    st.z_off = -r * (LP - 1);  // Z^T[d - r][r] at z_off + d LP
    st.wrow = lf_Wk + r * WSP;
    const float4 *ab = lf_Ab + 2 * (CX - r);  // step d: ab[2d], ab[2d + 1]
    const float *ib = lf_ila + (CX - r);      // step d: ib[d]
    ChainBlock c0, c1;
    chain_load<PV>(c0, st.wrow, ab, ib, 0);
    for (int t = 0; t < NBLK; t += 2) {
        chain_block<ZP, PV>(st, c0, c1, st.wrow, ab, ib, t);
        __syncthreads();
        chain_block<ZP, PV>(st, c1, c0, st.wrow, ab, ib, t + 1);
        __syncthreads();
    }
}

// Helper units stay in their factor rows.  A row-direction unit with anchor a
// takes, in the block whose first diagonal is D0, the LJ entries (x, a + p) of
// row x = D0 - a; their bulk runs over k < s0 - x = a - LJ against the rows
// LA[a + p][.].  x and D0 advance together, so the unit meets the same four
// factor rows and the same length in every block: it reads them once, into
// registers, with the entries at k >= a - LJ (and rows past the tile) set to
// zero, and per block reads only its E row.  A column-direction unit takes
// the entries (a + p, x) of column x = D0 - a, against LB[a + p][.] and the
// column Z[.][x] (row x of lf_Z).  The zeroed factor entries make masks
// unnecessary: E and Z are zeroed before the sweep, so an entry the chain may
// be writing during the block is zero or final, and it meets a zero factor
// entry either way.  Anchors a <= LJ have no bulk terms; their bulk slots keep
// the zeros they start with.
//
// A unit is 4 lanes; lane q takes k = 16 ch + 4 q .. + 3 of each 16-wide
// chunk ch, and a 4 x 4 DPP transpose-reduce leaves it entry q's total.  The
// units of one wave share a direction and a chunk count NCH: anchors
// 16 (NCH - 1) + 5 .. 16 NCH + 4, so one wave per (direction, NCH).  Within a
// block, chunk ch+1 is requested before chunk ch is multiplied (a scheduling
// barrier keeps that order: the LDS wait counter retires requests in order).
template <int NCH>
__device__ __forceinline__ void helper_sweep(const int dir, const int a, const int q) {
    const bool unit = a <= TB - 1;
    const int len = a - LJ;
    const float *F = dir ? lf_B : lf_A;
    float4 y[NCH][LJ];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int p = 0; p < LJ; ++p) {
            const int k0 = 16 * ch + 4 * q, row = min(a + p, TB - 1);
            float4 v = *reinterpret_cast<const float4 *>(F + row * LP + k0);
            const bool in = unit && a + p <= TB - 1;
            v.x = in && k0 < len ? v.x : 0.0f;
            v.y = in && k0 + 1 < len ? v.y : 0.0f;
            v.z = in && k0 + 2 < len ? v.z : 0.0f;
            v.w = in && k0 + 3 < len ? v.w : 0.0f;
            y[ch][p] = v;
        }
    const float *Xb = (dir ? lf_Z : lf_E) + 4 * q;
    const bool o1 = q & 1, o2 = q & 2;
    // kept rolled: unrolled, the sweep's code outgrows the instruction cache
    // that two CUs share, and the chain's loop is refetched every block
#pragma unroll 1
    for (int t = 0; t < NBLK; ++t) {
        const int x = LJ * (t + 1) - a;  // this block's row (column) of the unit
        if (t + 1 < NBLK && unit && x >= 0 && x < TB) {
            const float *X = Xb + x * LP;
            float acc[LJ];
#pragma unroll
            for (int p = 0; p < LJ; ++p) acc[p] = 0.0f;
            float4 xc[2];
            xc[0] = *reinterpret_cast<const float4 *>(X);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                if (ch + 1 < NCH) xc[(ch + 1) & 1] = *reinterpret_cast<const float4 *>(X + 16 * (ch + 1));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int p = 0; p < LJ; ++p) acc[p] = dot4(xc[ch & 1], y[ch][p], acc[p]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // 4 x 4 transpose-reduce over the unit: lane q ends with entry q's sum
            const float k0v = o1 ? acc[1] : acc[0], s0v = o1 ? acc[0] : acc[1];
            const float k1v = o1 ? acc[3] : acc[2], s1v = o1 ? acc[2] : acc[3];
            const float r0 = k0v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s0v), 0xB1, 0xF, 0xF, false));
            const float r1 = k1v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s1v), 0xB1, 0xF, 0xF, false));
            const float kv = o2 ? r1 : r0, sv = o2 ? r0 : r1;
            const float tot = kv + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sv), 0x4E, 0xF, 0xF, false));
            // entry q: (x, a + q) or (a + q, x); bulk slot [dir][its row][q]
            float *buf = lf_bulk + ((t + 1) & 1) * 2 * TB * LJ;
            float *dst = a + q <= TB - 1 ? buf + (dir * TB + (dir ? a + q : x)) * LJ + q
                                         : lf_sink + 2 * TB + (threadIdx.x & 63);
            *dst = tot;
        }
        __syncthreads();
    }
}

// helper waves w = 1..11 (wave w on SIMD w % 4; SIMD 0 also runs the chain):
// the two four-chunk classes on SIMDs 1 and 2, each beside a two-chunk class,
// the two three-chunk classes on SIMD 3, the one-chunk classes beside the
// chain; waves 9-11 only meet the barriers.
__device__ __forceinline__ void leaf_helpers(const int w, const int lane) {
    // (NCH - 1) * 2 + direction, or -1
    constexpr int kClass[12] = {-1, 6, 7, 4, 0, 2, 3, 5, 1, -1, -1, -1};
    const int cls = kClass[w];
    const int q = lane & 3;
    if (cls < 0) {
#pragma unroll 1
        for (int t = 0; t < NBLK; ++t) __syncthreads();
        return;
    }
    const int nch = (cls >> 1) + 1, dir = cls & 1;
    const int a = 16 * (nch - 1) + LJ + 1 + (lane >> 2);
    switch (nch) {
        case 1: helper_sweep<1>(dir, a, q); break;
        case 2: helper_sweep<2>(dir, a, q); break;
        case 3: helper_sweep<3>(dir, a, q); break;
        default: helper_sweep<4>(dir, a, q); break;
    }
}

// ------------------------------------------------------------ leaf push
// A recursion node over two tile diagonals [K, K+2) has a band update from
// diagonal K to K+1 alone.  It gets no launch: the leaf of diagonal K, which
// holds E(I,J), LA(J,J) and LB(I,I) in LDS and has prefetched LA(J+1,J) and
// LB(I+1,I), writes what its tile contributes to the next tile diagonal
// into the workspace:
//   Cd, to (I+1, J):  LB(I+1,I) U, U = E(I,J) LA(J,J)^T,
//   Cr, to (I, J+1):  V = E(I,J) LA(J+1,J)^T,
// and the leaf of diagonal K+1 applies them:
//   it subtracts Cd from its W tile as it loads it;
//   it applies LB(I,I) to V inside its own sweep: with V[r][c] added to the
//   row-direction sum of entry (r, c), that entry's z carries V[r][c] too,
//   so the column-direction sums subtract sum_{k<r} LB[r][k] V[k][c] and the
//   row term LB[r][r] V[r][c] -- together (LB(I,I) V)[r][c].
// U is the sweep's Z (each step forms z = E[r][c] LA[c][c] +
// sum_{k<c} E[r][k] LA[c][k]), which lf_Z already holds transposed, so two
// products remain.  They run on fp32 MFMA in 32 x 32 quadrants (waves 0-3,
// one per SIMD; lane l supplies row l % 32 of both operands and the k half
// l / 32), right after the sweep and beside the other waves' epilogue: they
// only read LDS that is final once the sweep has ended.

// acc += A[i][k] B[j][k]^T over k < KN for the 32 x 32 block; fa(i, k), fb(j, k)
// return the float4 at k .. k+3 of row i (j) of the block.
template <int KN, class FA, class FB>
__device__ __forceinline__ void mfma_block(floatx16 &acc, FA fa, FB fb) {
    const int lane = threadIdx.x & 63, i = lane & 31, k0 = (lane >> 5) * (KN / 2);
#pragma unroll
    for (int s4 = 0; s4 < KN / 8; ++s4) {
        const float4 av = fa(i, k0 + 4 * s4);
        const float4 bv = fb(i, k0 + 4 * s4);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv.z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv.w, acc, 0, 0, 0);
    }
}

__device__ __forceinline__ float4 lds4(const float *base, int stride, int row, int k) {
    return *reinterpret_cast<const float4 *>(base + row * stride + k);
}

// waves 0-3: quadrant (w >> 1, w & 1) of both contributions
__device__ __forceinline__ void leaf_push(const LeafArgs &a, int I, int J, int w) {
    const int lane = threadIdx.x & 63;
    const int qr = w >> 1, qc = w & 1;
    const bool down = I + 1 < a.M, right = J + 1 < a.N;
    const int64_t r0 = (int64_t)I * TB, c0 = (int64_t)J * TB;
    const int rb = 32 * qr, cb = 32 * qc;
    floatx16 acc, acc2;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = acc2[v] = 0.0f;
    if (down) {  // LB(I+1,I) U with U^T = Z^T
        auto fa = [&](int i, int k) { return lds4(lf_P + TB * GP, GP, rb + i, k); };
        auto fb = [&](int j, int k) { return lds4(lf_Z, LP, cb + j, k); };
        mfma_block<64>(acc, fa, fb);
    }
    if (right) {  // V = E LA(J+1,J)^T
        auto fa = [&](int i, int k) { return lds4(lf_E, LP, rb + i, k); };
        auto fb = [&](int j, int k) { return lds4(lf_P, GP, cb + j, k); };
        mfma_block<64>(acc2, fa, fb);
    }
    // accumulator: lane holds column lane % 32, register v row 8(v/4) + 4(lane/32) + v%4
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int64_t rr = rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3), cc = cb + (lane & 31);
        if (down) a.Cd[(r0 + TB + rr) * a.np + c0 + cc] = acc[v];
        if (right) a.Cr[(r0 + rr) * a.np + c0 + TB + cc] = acc2[v];
    }
}

// flags: LEAF_PULL apply the contributions pushed by the previous leaf;
// LEAF_PUSH compute this tile's contributions to the next tile diagonal.
// A leaf has at most one of them: a pulling leaf keeps the pushed V in the
// push operands' LDS (lf_P), which it does not otherwise use.
constexpr int LEAF_PULL = 1, LEAF_PUSH = 2;

template <bool ZP>
__global__ __launch_bounds__(LEAF_THREADS) void leaf_kernel(LeafArgs a, int K, int flags) {
    const int tid = threadIdx.x;
    const int Ilo = max(0, K - a.N + 1);
    const int I = Ilo + blockIdx.x;
    const int J = K - I;
    const int64_t r0 = (int64_t)I * TB, c0 = (int64_t)J * TB;

    const bool pull_up = (flags & LEAF_PULL) && I >= 1, pull_left = (flags & LEAF_PULL) && J >= 1;
    const bool push_right = (flags & LEAF_PUSH) && J + 1 < a.N, push_down = (flags & LEAF_PUSH) && I + 1 < a.M;
    // Every global read of the prologue is issued before the first LDS write,
    // so the tile's loads share one memory round trip: each thread reads its
    // float4 of every operand for at most two positions, and the row
    // parameters.  A leaf pulls or pushes, never both, so two extra operands
    // cover either case: x1 is Cd (pulling) or LA(J+1,J) (pushing), x2 is Cr
    // or LB(I+1,I).  The reads are unconditional (straight-line code keeps
    // them in flight together); an operand the leaf does not use is read from
    // its own W tile, and its value is discarded.
    static_assert(2 * LEAF_THREADS >= TB * 16 && LEAF_THREADS <= TB * 16, "two positions per thread");
    float s_ld = 1.0f, z_ld = 0.0f;
    if (tid < TB) {
        s_ld = a.sc[r0 + tid];
        z_ld = a.zp[r0 + tid];
    }
    struct PrologueLoads {
        float4 w, lb, la, x1, x2;
    };
    auto load_at = [&](int idx) {
        const int r = idx >> 4, c4 = (idx & 15) * 4;
        const int64_t g = (r0 + r) * a.np + c0 + c4;
        const int64_t gb = (r0 + r) * a.mp + r0 + c4, ga = (c0 + r) * a.np + c0 + c4;
        const float *x1 = pull_up ? a.Cd + g : push_right ? a.LAp + ga + TB * a.np : a.Wp + g;
        const float *x2 = pull_left ? a.Cr + g : push_down ? a.LBp + gb + TB * a.mp : a.Wp + g;
        PrologueLoads l;
        l.w = *reinterpret_cast<const float4 *>(a.Wp + g);
        l.lb = *reinterpret_cast<const float4 *>(a.LBp + gb);
        l.la = *reinterpret_cast<const float4 *>(a.LAp + ga);
        l.x1 = *reinterpret_cast<const float4 *>(x1);
        l.x2 = *reinterpret_cast<const float4 *>(x2);
        return l;
    };
    auto store_at = [&](int idx, const PrologueLoads &l) {
        const int r = idx >> 4, c4 = (idx & 15) * 4;
        float4 wv = l.w;
        if (pull_up) {
            wv.x -= l.x1.x; wv.y -= l.x1.y; wv.z -= l.x1.z; wv.w -= l.x1.w;
        }
        if (pull_left) {  // V, applied in the sweep; stored skewed like W
            float *vk = lf_P + r * WSP + r + c4;
            vk[0] = l.x2.x;
            vk[1] = l.x2.y;
            vk[2] = l.x2.z;
            vk[3] = l.x2.w;
        }
        float *wk = lf_Wk + r * WSP + r + c4;
        wk[0] = wv.x;
        wk[1] = wv.y;
        wk[2] = wv.z;
        wk[3] = wv.w;
        *reinterpret_cast<float4 *>(lf_B + r * LP + c4) = l.lb;
        *reinterpret_cast<float4 *>(lf_A + r * LP + c4) = l.la;
        if (push_right) *reinterpret_cast<float4 *>(lf_P + r * GP + c4) = l.x1;
        if (push_down) *reinterpret_cast<float4 *>(lf_P + (TB + r) * GP + c4) = l.x2;
    };
    const bool second = tid < TB * 16 - LEAF_THREADS;
    // the tile's column band table and row reciprocals (kept by threads < TB)
    const int q = tid & (TB - 1);
    float4 tb0, tb1;
    float tbi, ilb;
    if (tid < TB) {
        tb0 = a.tabA[2 * (c0 + q)];
        tb1 = a.tabA[2 * (c0 + q) + 1];
        tbi = a.tabI[c0 + q];
        ilb = a.ilb[r0 + q];
    }
    const PrologueLoads l0 = load_at(tid);
    PrologueLoads l1;
    if (second) l1 = load_at(tid + LEAF_THREADS);
    // while the loads are in flight: the LDS that starts at zero
    for (int idx = tid; idx < 2 * 2 * TB * LJ / 4; idx += LEAF_THREADS)
        reinterpret_cast<float4 *>(lf_bulk)[idx] = make_float4(0.f, 0.f, 0.f, 0.f);
    // E and Z: the helpers read entries the chain has not written yet
    for (int idx = tid; idx < TB * LP / 4; idx += LEAF_THREADS) {
        reinterpret_cast<float4 *>(lf_E)[idx] = make_float4(0.f, 0.f, 0.f, 0.f);
        reinterpret_cast<float4 *>(lf_Z)[idx] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the skewed W's (and V's) slots outside a row's 64 entries, so that an
    // off-tile step's pre-rounding value is finite and its error, scaled by the
    // zero reciprocal of an off-tile column, exactly zero: the 16 positions
    // (r, 4 j) of row r take its WSP - TB such slots k = j, j + 16, ...
    static_assert(WSP - TB <= 5 * 16, "five pad slots per position");
    auto zero_pad = [&](int idx) {
        const int r = idx >> 4, j = idx & 15;
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const int k = j + 16 * m;
            if (k < WSP - TB) {
                const int slot = r * WSP + (k < r ? k : k + TB);
                lf_Wk[slot] = 0.0f;
                if (pull_left) lf_P[slot] = 0.0f;
            }
        }
    };
    zero_pad(tid);
    if (second) zero_pad(tid + LEAF_THREADS);
    // the band table is zero outside the tile's columns
    for (int x = tid; x < NCX - TB; x += LEAF_THREADS) {
        const int xx = x < CX ? x : x + TB;
        lf_Ab[2 * xx] = make_float4(0.f, 0.f, 0.f, 0.f);
        lf_Ab[2 * xx + 1] = make_float4(0.f, 0.f, 0.f, 0.f);
        lf_ila[xx] = 0.0f;
    }
    store_at(tid, l0);
    if (second) store_at(tid + LEAF_THREADS, l1);
    if (tid < TB) {
        lf_Ab[2 * (CX + q)] = tb0;
        lf_Ab[2 * (CX + q) + 1] = tb1;
        lf_ila[CX + q] = tbi;
        lf_row[tid] = make_float4(s_ld, 1.0f / s_ld, z_ld, ilb);
    }
    __syncthreads();

    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (w == 0) {
        if (pull_left) leaf_chain<ZP, true>(tid, (float)a.qmin, (float)a.qmax);
        else leaf_chain<ZP, false>(tid, (float)a.qmin, (float)a.qmax);
    }
    else leaf_helpers(w, tid & 63);
    // waves 0-3 push (when the node asks for it) while the others write the
    // outputs; both only read LDS that the sweep has finalised
    const bool push = flags & LEAF_PUSH;
    if (push && w < 4) leaf_push(a, I, J, w);
    const int et = push ? tid - 4 * 64 : tid, en = push ? LEAF_THREADS - 4 * 64 : LEAF_THREADS;
    if (et >= 0) {
        const float *Es = lf_E;
        const float4 *s_row = lf_row;

        // E tile to the band-update buffer
        if (a.order == BAKRON_ORDER_LA_FIRST) {
            for (int idx = et; idx < TB * 16; idx += en) {
                const int r = idx >> 4, c4 = (idx & 15) * 4;
                *reinterpret_cast<float4 *>(a.Ebuf + (r0 + r) * a.np + c0 + c4) =
                    *reinterpret_cast<const float4 *>(Es + r * LP + c4);
            }
        } else {
            for (int idx = et; idx < TB * 16; idx += en) {
                const int c = idx >> 4, rr4 = (idx & 15) * 4;
                *reinterpret_cast<float4 *>(a.Ebuf + (c0 + c) * a.mp + r0 + rr4) =
                    make_float4(Es[(rr4 + 0) * LP + c], Es[(rr4 + 1) * LP + c],
                                Es[(rr4 + 2) * LP + c], Es[(rr4 + 3) * LP + c]);
            }
        }
        // caller-visible outputs
        int bad = 0;
        if (a.out_vec) {
            // groups of 4 columns: with ldo % 4 == 0 (and so n % 4 == 0) a group is
            // wholly inside or outside
            for (int idx = et; idx < TB * 16; idx += en) {
                const int r = idx >> 4, c4 = (idx & 15) * 4;
                const int64_t gi = r0 + r, gj = c0 + c4;
                const float4 e = *reinterpret_cast<const float4 *>(Es + r * LP + c4);
                bad |= (!isfinite(e.x) || !isfinite(e.y) || !isfinite(e.z) || !isfinite(e.w));
                if (gi < a.m && gj < a.n) {
                    const float *wk = lf_Wk + r * WSP + r + c4;
                    const float q0 = wk[0], q1 = wk[1], q2 = wk[2], q3 = wk[3];
                    const uint32_t packed = ((uint32_t)(uint8_t)(int8_t)(int)q0) |
                                            ((uint32_t)(uint8_t)(int8_t)(int)q1 << 8) |
                                            ((uint32_t)(uint8_t)(int8_t)(int)q2 << 16) |
                                            ((uint32_t)(uint8_t)(int8_t)(int)q3 << 24);
                    // the caller's outputs are not read again here: streaming stores
                    __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t *>(a.codes + gi * a.ldo + gj));
                    const float4 rc = s_row[r];
                    if (a.V) {
                        float *vp = a.V + gi * a.ldo + gj;
                        __builtin_nontemporal_store(rc.x * (q0 - rc.z), vp);
                        __builtin_nontemporal_store(rc.x * (q1 - rc.z), vp + 1);
                        __builtin_nontemporal_store(rc.x * (q2 - rc.z), vp + 2);
                        __builtin_nontemporal_store(rc.x * (q3 - rc.z), vp + 3);
                    }
                    if (a.E) {
                        float *ep = a.E + gi * a.ldo + gj;
                        __builtin_nontemporal_store(e.x, ep);
                        __builtin_nontemporal_store(e.y, ep + 1);
                        __builtin_nontemporal_store(e.z, ep + 2);
                        __builtin_nontemporal_store(e.w, ep + 3);
                    }
                }
            }
        } else {
            for (int idx = et; idx < TB * TB; idx += en) {
                const int r = idx >> 6, c = idx & 63;
                const int64_t gi = r0 + r, gj = c0 + c;
                bad |= !isfinite(Es[r * LP + c]);
                if (gi < a.m && gj < a.n) {
                    const float qf = lf_Wk[r * WSP + r + c];
                    const int8_t code = (int8_t)(int)qf;
                    a.codes[gi * a.ldo + gj] = code;
                    const float4 rc = s_row[r];
                    if (a.V) a.V[gi * a.ldo + gj] = rc.x * (qf - rc.z);
                    if (a.E) a.E[gi * a.ldo + gj] = Es[r * LP + c];
                }
            }
        }
        if (bad && a.dev_status) atomicOr(a.dev_status, BAKRON_DEV_NONFINITE);
    }
}

// -------------------------------------------------------------- band GEMMs
// C[ci][cj] (=|-=) sum_{kb=klo..khi} A[ci-block][kb-block] . B[cj-block][kb-block]^T
// on 64 x 64 tiles; both operands row-major with the contraction index
// contiguous.  The tile indices and the staircase K range of each output tile
// come from the recursion node (K, L, H):
//   mode 0  (LA first, product 1)  Tt(J',I) = sum_J LA(J',J) E(I,J)^T
//   mode 1  (LA first, product 2)  W(I',J') -= sum_I LB(I',I) Tt(J',I)^T
//   mode 2  (LB first, product 1)  S(I',J) = sum_I LB(I',I) Et(J,I)^T
//   mode 3  (LB first, product 2)  W(I',J') -= sum_J S(I',J) LA(J',J)^T
//   mode 4  dense: C(ci = rlo + y, cj = olo + x) over the K blocks 0 .. L-1,
//           cut at ci (H = 1: A lower triangular) or at cj (H = 2: B lower);
//           the cross update of a split solve
// Grid: x = offset along the band (from olo), y = row index (from rlo).
constexpr int BW_STORE = 0, BW_SUB = 1;  // BandArgs::subtract: C = acc, C -= acc
struct BandArgs {
    const float *A, *B;
    float *C;
    int64_t lda, ldb, ldc;
    int mode, K, L, H, M, N, rlo, subtract;
    int rows;  // output-tile rows of the launch (the grid pads them to a multiple of 8)
    int olo;   // band offset of the launch's first column (a launch may cover a sub-range)
    int cols;  // band offsets covered: olo .. olo + cols - 1
};

__device__ inline bool band_tile(const BandArgs &g, int bx, int by, int &ci, int &cj,
                                 int &klo, int &khi) {
    const int K = g.K, H = g.H, row = g.rlo + by, o = bx;
    if (g.mode == 0) {
        const int I = row, Jp = K - I + o;
        if (Jp < 0 || Jp >= g.N) return false;
        ci = Jp; cj = I; klo = max(0, K - I); khi = min(Jp, K + H - 1 - I);
    } else if (g.mode == 1) {
        const int Ip = row, Jp = K + H + o - Ip;
        if (Jp < 0 || Jp >= g.N) return false;
        ci = Ip; cj = Jp; klo = max(0, K - Jp); khi = min(Ip, K + H - 1);
    } else if (g.mode == 2) {
        const int J = row, Ip = K - J + o;
        if (Ip < 0 || Ip >= g.M) return false;
        ci = Ip; cj = J; klo = max(0, K - J); khi = min(Ip, K + H - 1 - J);
    } else if (g.mode == 3) {
        const int Ip = row, Jp = K + H + o - Ip;
        if (Jp < 0 || Jp >= g.N) return false;
        ci = Ip; cj = Jp; klo = max(0, K - Ip); khi = min(Jp, K + H - 1);
    } else {
        ci = row; cj = o; klo = 0;
        khi = H == 1 ? min(g.L - 1, ci) : (H == 2 ? min(g.L - 1, cj) : g.L - 1);
    }
    return klo <= khi;
}

// 256 threads = 4 waves; wave w owns the 32 x 32 quadrant (w/2, w%2) of the
// output tile and runs v_mfma_f32_32x32x2_f32.  Lane l supplies row l%32 of
// its A quadrant and row l%32 of its B quadrant; the two k slots of each
// instruction are k and k+32 of the 64-wide block (lanes 0-31 take the lower
// half, lanes 32-63 the upper), so every lane reads its operands as
// contiguous float4 from LDS.  The K block after next is prefetched into
// registers while the current one is multiplied (two register sets).
__global__ __launch_bounds__(256) void band_gemm_kernel(BandArgs g) {
    // Workgroups go to the 8 XCDs round-robin by linear id; XCD x takes the
    // rows y = x (mod 8), a whole row at a time, so the operand block that a
    // row shares (its A rows) is fetched into one XCD's L2 only.  Longest
    // tiles first: the K depth grows with the band offset in every mode and
    // with the row in the second products, so those run backwards.
    // The second products read, update and write back W tiles: there XCD x
    // takes the output tile rows I' = x (mod 8) in every launch, so the next
    // launch that updates a tile row runs on the XCD that holds it.
    const int lin = blockIdx.y * gridDim.x + blockIdx.x, slot = lin >> 3, x = lin & 7;
    const int gx = slot % (int)gridDim.x, k = slot / (int)gridDim.x;
    int by;
    if (g.mode == 1 || g.mode == 3) {
        by = g.rows - 1 - (((g.rlo + g.rows - 1 - x) % 8 + 8) % 8) - 8 * k;
        if (by < 0) return;
    } else {
        by = x + 8 * k;
        if (by >= g.rows) return;
    }
    const int bx = g.olo + gridDim.x - 1 - gx;
    int ci, cj, klo, khi;
    if (!band_tile(g, bx, by, ci, cj, klo, khi)) return;
    __shared__ __align__(16) float As[TB * GP];
    __shared__ __align__(16) float Bs[TB * GP];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr = w >> 1, wc = w & 1;
    const int lr = tid >> 4, lc = (tid & 15) * 4;
    const float *Ab = g.A + (int64_t)ci * TB * g.lda + (int64_t)lr * g.lda + lc;
    const float *Bb = g.B + (int64_t)cj * TB * g.ldb + (int64_t)lr * g.ldb + lc;
    const int64_t sa = 16 * g.lda, sb = 16 * g.ldb;
    // two register sets, each holding one K block's operands: block kb + 2 is
    // fetched while block kb is multiplied, so a load has two blocks' MFMA time
    // to arrive.  Past the last block the loads repeat it (always in bounds),
    // so every iteration issues the same loads and the waits stay static.
    float4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
    float4 xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3;
#define BK_GLOAD(kb, A0, A1, A2, A3, B0, B1, B2, B3)                                 \
    do {                                                                             \
        const float *a_ = Ab + (kb) * TB;                                            \
        const float *b_ = Bb + (kb) * TB;                                            \
        A0 = *reinterpret_cast<const float4 *>(a_);                                  \
        A1 = *reinterpret_cast<const float4 *>(a_ + sa);                             \
        A2 = *reinterpret_cast<const float4 *>(a_ + 2 * sa);                         \
        A3 = *reinterpret_cast<const float4 *>(a_ + 3 * sa);                         \
        B0 = *reinterpret_cast<const float4 *>(b_);                                  \
        B1 = *reinterpret_cast<const float4 *>(b_ + sb);                             \
        B2 = *reinterpret_cast<const float4 *>(b_ + 2 * sb);                         \
        B3 = *reinterpret_cast<const float4 *>(b_ + 3 * sb);                         \
    } while (0)
#define BK_LSTORE(A0, A1, A2, A3, B0, B1, B2, B3)                                    \
    do {                                                                             \
        *reinterpret_cast<float4 *>(as_w) = A0;                                      \
        *reinterpret_cast<float4 *>(as_w + 16 * GP) = A1;                            \
        *reinterpret_cast<float4 *>(as_w + 32 * GP) = A2;                            \
        *reinterpret_cast<float4 *>(as_w + 48 * GP) = A3;                            \
        *reinterpret_cast<float4 *>(bs_w) = B0;                                      \
        *reinterpret_cast<float4 *>(bs_w + 16 * GP) = B1;                            \
        *reinterpret_cast<float4 *>(bs_w + 32 * GP) = B2;                            \
        *reinterpret_cast<float4 *>(bs_w + 48 * GP) = B3;                            \
    } while (0)
#define BK_MFMA()                                                                    \
    do {                                                                             \
        _Pragma("unroll") for (int s4 = 0; s4 < 8; ++s4) {                           \
            const float4 av = *reinterpret_cast<const float4 *>(ap + 4 * s4);        \
            const float4 bv = *reinterpret_cast<const float4 *>(bp + 4 * s4);        \
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.x, bv.x, acc, 0, 0, 0);    \
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.y, bv.y, acc, 0, 0, 0);    \
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.z, bv.z, acc, 0, 0, 0);    \
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av.w, bv.w, acc, 0, 0, 0);    \
        }                                                                            \
    } while (0)
    BK_GLOAD(klo, ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3);
    BK_GLOAD(min(klo + 1, khi), xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3);
    // accumulator layout of the 32 x 32 MFMA: lane l holds column l % 32;
    // register v holds row 8 (v / 4) + 4 (l / 32) + v % 4.  The old values of
    // a subtracted tile are loaded now, so their latency overlaps the K loop.
    float *cb = g.C + (int64_t)(ci * TB + wr * 32 + 4 * (lane >> 5)) * g.ldc + (int64_t)cj * TB +
                wc * 32 + (lane & 31);
    float old[16];
    if (g.subtract) {
#pragma unroll
        for (int v = 0; v < 16; ++v) old[v] = cb[(int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc];
    }
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    const float *ap = As + (wr * 32 + (lane & 31)) * GP + 32 * (lane >> 5);
    const float *bp = Bs + (wc * 32 + (lane & 31)) * GP + 32 * (lane >> 5);
    float *as_w = As + lr * GP + lc;
    float *bs_w = Bs + lr * GP + lc;
    for (int kb = klo;; kb += 2) {
        __syncthreads();
        BK_LSTORE(ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3);
        __syncthreads();
        BK_GLOAD(min(kb + 2, khi), ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3);
        BK_MFMA();
        if (kb + 1 > khi) break;
        __syncthreads();
        BK_LSTORE(xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3);
        __syncthreads();
        BK_GLOAD(min(kb + 3, khi), xa0, xa1, xa2, xa3, xb0, xb1, xb2, xb3);
        BK_MFMA();
        if (kb + 2 > khi) break;
    }
#undef BK_GLOAD
#undef BK_LSTORE
#undef BK_MFMA
    if (g.subtract) {
#pragma unroll
        for (int v = 0; v < 16; ++v) cb[(int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc] = old[v] - acc[v];
    } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) cb[(int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc] = acc[v];
    }
}

// Band products that run beside the leaves.  A launch has at most SIDE_WG
// (or SIDE_WG_QUARTER) workgroups of 1024 threads, and each workgroup's LDS
// (four tiles' operand blocks, 139 KB) keeps it alone on its CU, so a side
// launch leaves at least 64 CUs to the leaves (one workgroup of 160 KB LDS
// per tile; a tile diagonal of up to 64 tiles finds them empty).  The four
// 4-wave slots of a workgroup work independently, like four workgroups of
// band_gemm_kernel.  The launch's tiles, in band_gemm_kernel's grid order
// (row-major, longest first), form SIDE_QUEUES queues: queue x holds the rows
// y = x (mod SIDE_QUEUES), row after row.  Workgroup b works on queue
// b mod SIDE_QUEUES (linear workgroup ids reach the 8 XCDs round-robin, so a
// queue's rows, which share their A operand blocks, stay in one XCD's L2):
// its first tiles are dealt to slot 0 of every workgroup of that queue, then
// slot 1, and so on; after that a slot takes the next tile of its queue from
// the queue's counter, and once its queue is empty, from the next queues in
// turn (counters `ctr`, zero at the start).  A slot runs each tile exactly as
// band_gemm_kernel does, with a barrier of its own four waves (a counter in
// LDS) in place of the workgroup barrier.  A slot barrier waits for the three
// other waves of the slot, which run the same sequence of barriers; the wait
// is bounded all the same, and a wait that reaches the bound sets
// BAKRON_DEV_SPIN_LIMIT in *dev_status.
constexpr int SIDE_WG = 160;
// Shapes whose plan keeps a quarter of each wide node critical defer less per
// leaf; their side launches take more CUs (measured at 4096 x 4096: 160 ->
// 6.23 ms, 176 -> 6.19, 192 -> 6.18, 208 -> 6.28).  Shapes that keep half
// stay at SIDE_WG (11008 x 4096: 17.8 ms with 160, 18.0 with 192).
constexpr int SIDE_WG_QUARTER = 192;
constexpr int SIDE_THREADS = 1024;
constexpr int SIDE_QUEUES = 8;  // tile queues (and counters) of one side launch
constexpr int SPIN_LIMIT = 1 << 22;

__global__ __launch_bounds__(SIDE_THREADS) void band_side_kernel(BandArgs g, int *ctr,
                                                                 int32_t *dev_status) {
    __shared__ __align__(16) float As[4 * TB * GP];
    __shared__ __align__(16) float Bs[4 * TB * GP];
    __shared__ int s_arrive[4];  // arrivals at slot barriers, per slot
    __shared__ int s_tile[4];    // next tile index, per slot
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, q = w >> 2, wq = w & 3;
    const int wr = wq >> 1, wc = wq & 1;
    const int t2 = tid & 255, lr = t2 >> 4, lc = (t2 & 15) * 4;
    const int ntile = g.cols * g.rows;
    const float *ap = As + q * TB * GP + (wr * 32 + (lane & 31)) * GP + 32 * (lane >> 5);
    const float *bp = Bs + q * TB * GP + (wc * 32 + (lane & 31)) * GP + 32 * (lane >> 5);
    float *as_w = As + q * TB * GP + lr * GP + lc;
    float *bs_w = Bs + q * TB * GP + lr * GP + lc;
    // queue x: rows x, x + SIDE_QUEUES, ...; its workgroups b = x (mod SIDE_QUEUES)
    // deal its first 4 * (their number) tiles before its counter is used
    const int x = blockIdx.x % SIDE_QUEUES, lb = blockIdx.x / SIDE_QUEUES;
    auto qcount = [&](int qq) { return qq < g.rows ? (g.rows - qq + SIDE_QUEUES - 1) / SIDE_QUEUES * g.cols : 0; };
    auto qfirst = [&](int qq) { return 4 * (((int)gridDim.x - qq + SIDE_QUEUES - 1) / SIDE_QUEUES); };
    auto qtile = [&](int qq, int i) { return (qq + SIDE_QUEUES * (i / g.cols)) * g.cols + i % g.cols; };
    auto take = [&]() {  // the next tile from the queues, from this workgroup's own on
        for (int k = 0; k < SIDE_QUEUES; ++k) {
            const int qq = (x + k) % SIDE_QUEUES, cnt = qcount(qq), f = qfirst(qq);
            if (f >= cnt) continue;
            const int i = f + atomicAdd(ctr + qq, 1);
            if (i < cnt) return qtile(qq, i);
        }
        return ntile;
    };
    if (tid < 4) s_arrive[tid] = 0;
    __syncthreads();  // the only barrier of the whole workgroup
    int target = 0, stuck = 0;
    auto slot_barrier = [&]() {
        target += 4;
        if (lane == 0) __hip_atomic_fetch_add(&s_arrive[q], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (int spin = 0; __hip_atomic_load(&s_arrive[q], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target;
             ++spin) {
            if (spin >= SPIN_LIMIT) {
                stuck = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    };
    // the slot's first tile: dealt, or (uniformly over the slot) taken from the queues
    const int i0 = q * ((int)(gridDim.x - x + SIDE_QUEUES - 1) / SIDE_QUEUES) + lb;
    int t = i0 < qcount(x) ? qtile(x, i0) : -1;
    if (t < 0) {
        if (wq == 0 && lane == 0) s_tile[q] = take();
        slot_barrier();
        t = s_tile[q];
        slot_barrier();  // every wave has read s_tile[q] before it is written again
    }
    while (t < ntile) {
        int next = 0;
        if (wq == 0 && lane == 0) next = take();  // published after this tile
        const int gy = t / g.cols, gx = t - gy * g.cols;
        const int bx = g.olo + g.cols - 1 - gx;
        const int by = (g.mode == 1 || g.mode == 3) ? g.rows - 1 - gy : gy;
        int ci, cj, klo, khi;
        if (band_tile(g, bx, by, ci, cj, klo, khi)) {  // uniform over the slot
            const float *Ab = g.A + (int64_t)ci * TB * g.lda + (int64_t)lr * g.lda + lc;
            const float *Bb = g.B + (int64_t)cj * TB * g.ldb + (int64_t)lr * g.ldb + lc;
            const int64_t sa = 16 * g.lda, sb = 16 * g.ldb;
            float4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define BK_SLOAD(kb)                                                                 \
    do {                                                                             \
        const float *a_ = Ab + (kb) * TB;                                            \
        const float *b_ = Bb + (kb) * TB;                                            \
        ra0 = *reinterpret_cast<const float4 *>(a_);                                 \
        ra1 = *reinterpret_cast<const float4 *>(a_ + sa);                            \
        ra2 = *reinterpret_cast<const float4 *>(a_ + 2 * sa);                        \
        ra3 = *reinterpret_cast<const float4 *>(a_ + 3 * sa);                        \
        rb0 = *reinterpret_cast<const float4 *>(b_);                                 \
        rb1 = *reinterpret_cast<const float4 *>(b_ + sb);                            \
        rb2 = *reinterpret_cast<const float4 *>(b_ + 2 * sb);                        \
        rb3 = *reinterpret_cast<const float4 *>(b_ + 3 * sb);                        \
    } while (0)
            BK_SLOAD(klo);
            floatx16 acc;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
            for (int kb = klo; kb <= khi; ++kb) {
                slot_barrier();
                *reinterpret_cast<float4 *>(as_w) = ra0;
                *reinterpret_cast<float4 *>(as_w + 16 * GP) = ra1;
                *reinterpret_cast<float4 *>(as_w + 32 * GP) = ra2;
                *reinterpret_cast<float4 *>(as_w + 48 * GP) = ra3;
                *reinterpret_cast<float4 *>(bs_w) = rb0;
                *reinterpret_cast<float4 *>(bs_w + 16 * GP) = rb1;
                *reinterpret_cast<float4 *>(bs_w + 32 * GP) = rb2;
                *reinterpret_cast<float4 *>(bs_w + 48 * GP) = rb3;
                slot_barrier();
                if (kb < khi) BK_SLOAD(kb + 1);
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
#undef BK_SLOAD
            const int col = lane & 31;
            float *cb = g.C + (int64_t)(ci * TB + wr * 32 + 4 * (lane >> 5)) * g.ldc +
                        (int64_t)cj * TB + wc * 32 + col;
            if (g.subtract) {
                float old[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) old[v] = cb[(int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc];
#pragma unroll
                for (int v = 0; v < 16; ++v) cb[(int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc] = old[v] - acc[v];
            } else {
#pragma unroll
                for (int v = 0; v < 16; ++v) cb[(int64_t)(8 * (v >> 2) + (v & 3)) * g.ldc] = acc[v];
            }
        }
        // every wave of the slot has read s_tile[q] and finished its LDS reads
        // of this tile; then the next index is published
        slot_barrier();
        if (wq == 0 && lane == 0) s_tile[q] = next;
        slot_barrier();
        t = s_tile[q];
    }
    if (stuck && lane == 0 && dev_status) atomicOr(dev_status, BAKRON_DEV_SPIN_LIMIT);
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int *p, int n) {
    for (int k = blockIdx.x * 256 + threadIdx.x; k < n; k += gridDim.x * 256) p[k] = 0;
}

// ----------------------------------------------------------------- finalise
__global__ __launch_bounds__(256) void sumsq_partial_kernel(const float *__restrict__ x,
                                                            int64_t count, double *partial) {
    __shared__ double red[256];
    const int64_t chunk = (count + NPART - 1) / NPART;
    const int64_t beg = blockIdx.x * chunk;
    const int64_t end = min(count, beg + chunk);
    double s = 0.0;
    int64_t k = beg + threadIdx.x;
    for (; k + 7 * 256 < end; k += 8 * 256) {  // eight loads in flight; the same order of the sum
        float xv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) xv[u] = x[k + u * 256];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const double v = xv[u];
            s += v * v;
        }
    }
    for (; k < end; k += 256) {
        const double v = x[k];
        s += v * v;
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void sumsq_final_kernel(const double *partial, double *out) {
    __shared__ double red[256];
    double s = 0.0;
    for (int k = threadIdx.x; k < NPART; k += 256) s += partial[k];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = red[0];
}

// ------------------------------------------------------- BaKron-antidiagonal
// The comparison variant of the pages (pith.science review of arXiv
// 2608.06291, "If this is right": BaKron runs about 27x faster than it at
// 4096 x 4096; "Core claim": all variants give the same output).  Every entry
// anti-diagonal d is rounded at once, then its rank-|d| update is applied to
// the rest of the matrix:
//   W[i'][j'] -= sum over the entries (i, j) of d of LB[i'][i] e_ij LA[j'][j].
// The per-entry rounding is the leaf's, operation for operation.

// Rounds the entries (i, d - i), i = i_min .. i_min + cnt - 1; e to eb[i - i_min].
template <bool ZP>
__global__ __launch_bounds__(256) void ad_round_kernel(
    const float *__restrict__ Wp, const float *__restrict__ LAp, const float *__restrict__ LBp,
    const float *__restrict__ sc, const float *__restrict__ zp, int64_t mp, int64_t np, int64_t n,
    int d, int i_min, int cnt, float qminf, float qmaxf, int8_t *__restrict__ codes,
    float *__restrict__ V, float *__restrict__ E, float *__restrict__ eb, int32_t *dev_status) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= cnt) return;
    const int64_t i = i_min + k, j = d - i;
    const float P = Wp[i * np + j];
    const float s = sc[i], rs = 1.0f / s, z = zp[i];
    float qz, res;
    if (ZP) {
        qz = __builtin_amdgcn_fmed3f(rintf(P * rs) + z, qminf, qmaxf);
        res = fmaf(-s, qz - z, P);
    } else {
        qz = __builtin_amdgcn_fmed3f(rintf(P * rs), qminf, qmaxf);
        res = fmaf(-s, qz, P);
    }
    const float e = res * ((1.0f / LBp[i * mp + i]) * (1.0f / LAp[j * np + j]));
    eb[k] = e;
    codes[i * n + j] = (int8_t)(int)qz;
    if (V) V[i * n + j] = s * (qz - z);
    if (E) E[i * n + j] = e;
    if (!isfinite(e) && dev_status) atomicOr(dev_status, BAKRON_DEV_NONFINITE);
}

// The rank-cnt update of diagonal d on the 64 x 64 output tiles of W from tile
// row i_min / 64 and tile column (d - i_min - cnt + 1) / 64 on (rows above the
// diagonal's first row and columns left of its first column get exact zeros:
// LB and LA are lower triangular), skipping tiles that lie on or before d.
// C[i'][j'] -= sum_k A[i'][k] B[j'][k], A[i'][k] = LB[i'][i_min + k],
// B[j'][k] = e_k LA[j'][d - i_min - k], k in chunks of 64 (zero past cnt);
// fp32 MFMA as in band_gemm_kernel.
__global__ __launch_bounds__(256) void ad_update_kernel(
    float *__restrict__ Wp, const float *__restrict__ LAp, const float *__restrict__ LBp,
    const float *__restrict__ eb, int64_t mp, int64_t np, int d, int i_min, int cnt, int ti0,
    int tj0) {
    const int ti = ti0 + blockIdx.y, tj = tj0 + blockIdx.x;
    if (TB * (ti + tj) + 2 * (TB - 1) <= d) return;  // every entry of the tile is at or before d
    __shared__ __align__(16) float As[TB * GP];
    __shared__ __align__(16) float Bs[TB * GP];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr = w >> 1, wc = w & 1;
    const int lr = tid >> 4, lc = (tid & 15) * 4;
    floatx16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    const float *ap = As + (wr * 32 + (lane & 31)) * GP + 32 * (lane >> 5);
    const float *bp = Bs + (wc * 32 + (lane & 31)) * GP + 32 * (lane >> 5);
    for (int kc = 0; kc < cnt; kc += TB) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = lr + 16 * q;
            const int64_t gi = (int64_t)ti * TB + r, gj = (int64_t)tj * TB + r;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int k = kc + lc + t;
                float a = 0.0f, b = 0.0f;
                if (k < cnt) {
                    a = LBp[gi * mp + i_min + k];
                    b = eb[k] * LAp[gj * np + (d - i_min - k)];
                }
                As[r * GP + lc + t] = a;
                Bs[r * GP + lc + t] = b;
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
    float *cb = Wp + (int64_t)(ti * TB + wr * 32 + 4 * (lane >> 5)) * np + (int64_t)tj * TB + wc * 32 + col;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        float *c = cb + (int64_t)(8 * (v >> 2) + (v & 3)) * np;
        *c = *c - acc[v];
    }
}

// ---------------------------------------------------------------- schedule
struct Node {
    int leaf;  // 1: leaf(K); 0: band(K, L, H)
    int flags;  // leaf only: LEAF_PUSH / LEAF_PULL (two-diagonal nodes run inside the leaves)
    int K, L, H;
    int depth;  // band only: recursion depth (the top node is 0)
    int slab;   // band only: its T buffer (set by build_plan)
};

void build_nodes(int K, int L, std::vector<Node> &out, int depth = 0) {
    if (L == 1) {
        out.push_back({1, 0, K, 1, 0, depth, 0});
        return;
    }
    if (L == 2) {  // leaf(K), band(K, 2, 1), leaf(K+1): the band runs inside the two leaves
        out.push_back({1, LEAF_PUSH, K, 1, 0, depth, 0});
        out.push_back({1, LEAF_PULL, K + 1, 1, 0, depth, 0});
        return;
    }
    const int H = L / 2;  // split of the range [K, K+L) at K + floor(L/2)
    build_nodes(K, H, out, depth + 1);
    out.push_back({0, 0, K, L, H, depth, 0});
    build_nodes(K + H, L - H, out, depth + 1);
}

int depth_of(int L) {
    int d = 0;
    while (L > 1) {
        L = L - L / 2;
        ++d;
    }
    return d;
}

// row range and grid of one band product
struct Launch {
    int mode, rlo, rows, cols;
};

void band_launches(int order, int K, int L, int H, int M, int N, Launch &p1, Launch &p2) {
    if (order == BAKRON_ORDER_LA_FIRST) {
        p1.mode = 0;
        p1.rlo = std::max(0, K - N + 1);
        p1.rows = std::min(M - 1, K + H - 1) - p1.rlo + 1;
        p1.cols = L;
        p2.mode = 1;
    } else {
        p1.mode = 2;
        p1.rlo = std::max(0, K - M + 1);
        p1.rows = std::min(N - 1, K + H - 1) - p1.rlo + 1;
        p1.cols = L;
        p2.mode = 3;
    }
    p2.rlo = std::max(0, K + H - N + 1);
    p2.rows = std::min(M - 1, K + L - 1) - p2.rlo + 1;
    p2.cols = L - H;
}

// ------------------------------------------------------------------- plan
// The order of a solve's work on two streams.  The critical stream runs the
// leaves in diagonal order and, for every band node, the products that feed
// its first target diagonals.  A node whose right part spans R = L - H >=
// SIDE_MIN_R diagonals keeps only the targets K + H .. a - 1, a = K + H +
// (R >> shift) (R >> 1 below 2 SIDE_MIN_R), critical: its first product over the T diagonals from a
// on and its second product over the targets from a on go to the side stream.
// They are forked by events once their inputs exist (the sources are final
// when the node starts; the second product also reads the critical part of T)
// and joined before the first critical step that updates or reads their
// targets: the leaf of diagonal a, or a band node whose targets reach a.  So
// the deferred products run while the leaves of K + H .. a - 1 hold a few CUs.
// A node that defers keeps T in the buffer of its recursion depth until its
// deferred products are joined, which happens inside its right subtree, before
// the next node of that depth starts; so a deferred product shares no T tile
// with the nodes that run meanwhile.  Nodes below the deepest level that
// defers run both products back to back on the critical stream and share one
// more buffer: a solve needs (that level + 2) T buffers.  On one stream the
// same plan gives the same results bit for bit.
constexpr int OP_LEAF = 0, OP_BAND = 1, OP_RECORD = 2, OP_WAIT = 3;
constexpr int SIDE_MIN_R = 16;
constexpr int PREP_TILES = 16;  // tile rows / columns the critical stream sets up itself
// A node with R < 2 SIDE_MIN_R keeps half of its targets critical whatever the
// shift: a quarter would leave its deferred products only R/4 leaves to run
// beside, and the critical stream would wait for them (measured at 4096 x 4096:
// 5.683 -> 5.639 ms with half).
// The deferred work should fit beside the leaves: the side kernel sustains
// about 48 TFLOP/s on its CUs and a leaf launch lasts about 25 us, so about
// 1.2e9 flops per leaf launch.  A shape keeps a quarter of each wide node's
// targets critical (shift 2) if that defers no more than this, else half
// (shift 1).  Measured: 4096 x 4096 defers 0.77e9 per leaf with shift 2 and
// runs faster than with shift 1; 11008 x 4096 and 4096 x 14336 defer 2.1e9
// and 3.0e9 with shift 2 and run 5 % and 9 % faster with shift 1.
constexpr double SIDE_BUDGET = 1.2e9;

struct Op {
    int kind;
    int side;  // OP_BAND: deferred product; OP_RECORD / OP_WAIT: 1 = on the side stream
    int ev;    // OP_RECORD / OP_WAIT: event index
    Node nd;   // OP_LEAF / OP_BAND
    int prod;  // OP_BAND: 0 = first product (T diagonals lo .. hi-1), 1 = second (targets lo .. hi-1)
    int lo, hi;
};

struct Plan {
    std::vector<Op> ops;
    int events = 0;
    int slabs = 1;  // T buffers
};

Plan build_plan(int M, int N, int shift) {
    Plan pl;
    std::vector<Node> nodes;
    build_nodes(0, M + N - 1, nodes);
    int shared = 0;  // one past the deepest level with a deferring node
    for (const Node &nd : nodes)
        if (!nd.leaf && nd.L - nd.H >= SIDE_MIN_R) shared = std::max(shared, nd.depth + 1);
    for (Node &nd : nodes) nd.slab = std::min(nd.depth, shared);
    pl.slabs = shared + 1;
    std::vector<std::pair<int, int>> pending;  // (first target diagonal, completion event)
    auto join = [&](int upto) {  // the critical stream waits for deferred targets below upto
        for (size_t k = 0; k < pending.size();) {
            if (pending[k].first < upto) {
                pl.ops.push_back(Op{OP_WAIT, 0, pending[k].second, Node{}, 0, 0, 0});
                pending.erase(pending.begin() + (std::ptrdiff_t)k);
            } else {
                ++k;
            }
        }
    };
    auto band = [&](const Node &nd, int side, int prod, int lo, int hi) {
        pl.ops.push_back(Op{OP_BAND, side, -1, nd, prod, lo, hi});
    };
    // A fork's side-stream steps are issued after the next leaf: the dependences
    // are the same, and a captured graph then creates the leaf's node before the
    // side branch's.
    std::vector<Op> forked;
    auto fork = [&](int ev) {
        pl.ops.push_back(Op{OP_RECORD, 0, ev, Node{}, 0, 0, 0});
        forked.push_back(Op{OP_WAIT, 1, ev, Node{}, 0, 0, 0});
    };
    for (const Node &nd : nodes) {
        if (nd.leaf) {
            join(nd.K + 1);
            pl.ops.push_back(Op{OP_LEAF, 0, -1, nd, 0, 0, 0});
            pl.ops.insert(pl.ops.end(), forked.begin(), forked.end());
            forked.clear();
            continue;
        }
        const int R = nd.L - nd.H, end = nd.K + nd.L;
        const int keep = R >= SIDE_MIN_R ? (R >> (R < 2 * SIDE_MIN_R ? 1 : shift)) : R;
        if (keep < R) {
            const int a = nd.K + nd.H + keep;
            const int e1 = pl.events++, e3 = pl.events++;
            band(nd, 0, 0, nd.K, a);
            join(a);
            band(nd, 0, 1, nd.K + nd.H, a);
            fork(e1);  // after the critical products: the deferred ones run beside the next leaves
            forked.push_back(Op{OP_BAND, 1, -1, nd, 0, a, end});
            forked.push_back(Op{OP_BAND, 1, -1, nd, 1, a, end});
            forked.push_back(Op{OP_RECORD, 1, e3, Node{}, 0, 0, 0});
            pending.push_back({a, e3});
        } else {
            band(nd, 0, 0, nd.K, end);
            join(end);
            band(nd, 0, 1, nd.K + nd.H, end);
        }
    }
    pl.ops.insert(pl.ops.end(), forked.begin(), forked.end());
    join(INT_MAX);
    return pl;
}

// Launch geometry of one band op of the plan; false when it holds no tile.
// Grid column o of a product covers band diagonal base + o; a row r meets the
// columns lo .. hi-1 when the tile's other index, diagonal - r, can lie in
// 0 .. X-1.
bool band_geometry(const Op &op, int order, int M, int N, int &mode, int &olo, int &cols,
                   int &rlo, int &rows) {
    Launch p1, p2;
    band_launches(order, op.nd.K, op.nd.L, op.nd.H, M, N, p1, p2);
    const Launch &p = op.prod ? p2 : p1;
    mode = p.mode;
    olo = op.lo - (op.prod ? op.nd.K + op.nd.H : op.nd.K);
    cols = op.hi - op.lo;
    const int X = (mode == 2) ? M : N;
    rlo = std::max(p.rlo, op.lo - X + 1);
    rows = std::min(p.rlo + p.rows - 1, op.hi - 1) - rlo + 1;
    return cols > 0 && rows > 0;
}


// Flops of the band-GEMM launches of one order (host mirror of band_tile),
// over the plan's band ops: exec counts every dense 64 x 64 x 64 tile step;
// useful leaves out the zero half of a triangular diagonal factor block (LA(J,J)
// or LB(I,I)).  The side_* fields count the deferred products alone.
struct BandCount {
    double exec, useful;
    int launches;
    double side_exec, side_useful;
    int side_launches;
};

BandCount band_flops(const Plan &pl, int order, int M, int N) {
    BandCount c{};
    const double tile = 2.0 * TB * TB * TB, dtile = 2.0 * TB * TB * (TB + 1) / 2;
    for (const Op &op : pl.ops) {
        int mode, olo, cols, rlo, rows;
        if (op.kind != OP_BAND || !band_geometry(op, order, M, N, mode, olo, cols, rlo, rows)) continue;
        const int K = op.nd.K, H = op.nd.H;
        double full = 0, diag = 0;
        for (int row = rlo; row < rlo + rows; ++row)
            for (int o = olo; o < olo + cols; ++o) {
                int lo, hi, fac;  // fac: k block holding the factor's diagonal block
                if (mode == 0) {
                    const int Jp = K - row + o;
                    if (Jp < 0 || Jp >= N) continue;
                    lo = std::max(0, K - row); hi = std::min(Jp, K + H - 1 - row); fac = Jp;
                } else if (mode == 2) {
                    const int Ip = K - row + o;
                    if (Ip < 0 || Ip >= M) continue;
                    lo = std::max(0, K - row); hi = std::min(Ip, K + H - 1 - row); fac = Ip;
                } else {
                    const int Jp = K + H + o - row;
                    if (Jp < 0 || Jp >= N) continue;
                    if (mode == 1) { lo = std::max(0, K - Jp); hi = std::min(row, K + H - 1); fac = row; }
                    else { lo = std::max(0, K - row); hi = std::min(Jp, K + H - 1); fac = Jp; }
                }
                if (hi < lo) continue;
                full += hi - lo + 1;
                if (fac >= lo && fac <= hi) diag += 1;
            }
        const double ex = full * tile, us = (full - diag) * tile + diag * dtile;
        c.exec += ex;
        c.useful += us;
        c.launches += 1;
        if (op.side) {
            c.side_exec += ex;
            c.side_useful += us;
            c.side_launches += 1;
        }
    }
    return c;
}

// Two-diagonal nodes: the update of each target tile is two dense
// 64 x 64 x 64 products (LB E LA^T); the leaves run them as one MFMA product
// each (U comes from the sweep, and LB(I,I) V is applied inside the next sweep).
void pull_counts(int M, int N, double *flops, int *leaves) {
    std::vector<Node> nodes;
    build_nodes(0, M + N - 1, nodes);
    double f = 0;
    int nl = 0;
    for (const Node &nd : nodes) {
        if (!nd.leaf || !(nd.flags & LEAF_PUSH)) continue;
        ++nl;
        for (int I = std::max(0, nd.K - N + 1); I <= std::min(M - 1, nd.K); ++I) {
            const int J = nd.K - I;
            f += (I + 1 < M ? 2 : 0) + (J + 1 < N ? 2 : 0);
        }
    }
    *flops = f * 2.0 * TB * TB * TB;
    *leaves = nl;
}

// Algorithm 6 at single anti-diagonal granularity (product order LA first):
// per node [k, k+l) split at h, T = E_S LA^T over the band and LB T on R.
double algorithmic_band_flops(int64_t m, int64_t n) {
    struct Frame { int64_t k, l; };
    std::vector<Frame> stack{{0, m + n - 1}};
    double macs = 0;
    while (!stack.empty()) {
        const Frame f = stack.back();
        stack.pop_back();
        if (f.l <= 1) continue;
        const int64_t k = f.k, l = f.l, h = l / 2;
        stack.push_back({k, h});
        stack.push_back({k + h, l - h});
        // T rows i with a source in S; columns jj of the band that some target
        // row consumes (entries on S diagonals only if a row below reaches R);
        // count_J = min(jj, b) - a + 1 per entry
        const int64_t ilo = std::max<int64_t>(0, k - n + 1), ihi = std::min<int64_t>(m - 1, k + h - 1);
        for (int64_t i = ilo; i <= ihi; ++i) {
            const int64_t a = std::max<int64_t>(0, k - i);
            const int64_t b = std::min<int64_t>(n - 1, k + h - 1 - i);
            const int64_t c = std::min<int64_t>(n - 1, k + l - 1 - i);
            if (b < a) continue;
            const int64_t p0 = std::max<int64_t>(a, k + h - m + 1);
            if (p0 <= b)
                macs += (double)(b - p0 + 1) * (double)(p0 + b) / 2.0 - (double)(a - 1) * (double)(b - p0 + 1);
            macs += (double)(c - b) * (double)(b - a + 1);
        }
        // targets (i2, jj) in R: count_I = min(i2, k+h-1) - max(0, k-jj) + 1
        for (int64_t jj = 0; jj < n; ++jj) {
            const int64_t lo = std::max<int64_t>(0, k + h - jj);
            const int64_t hi = std::min<int64_t>(m - 1, k + l - 1 - jj);
            if (hi < lo) continue;
            const int64_t al = std::max<int64_t>(0, k - jj), be = k + h - 1;
            const int64_t p = std::min(hi, be);
            if (lo <= p) macs += (double)(p - lo + 1) * (double)(lo + p) / 2.0 - (double)(al - 1) * (double)(p - lo + 1);
            const int64_t q = std::max(lo, be + 1);
            if (q <= hi) macs += (double)(hi - q + 1) * (double)(be - al + 1);
        }
    }
    return 2.0 * macs;
}

struct ShapeInfo {
    BandCount band[3];  // index by order (1, 2)
    double pull_flops;
    int pull_leaves;
    int auto_order;
    Plan plan;
    int side_ops;     // deferred products of the plan (one tile counter each)
    int side_wg;      // workgroups of a side launch
};

std::mutex g_shape_mu;
std::map<std::pair<int, int>, ShapeInfo> g_shapes;

const ShapeInfo &shape_info(int M, int N) {
    std::lock_guard<std::mutex> lock(g_shape_mu);
    auto key = std::make_pair(M, N);
    auto it = g_shapes.find(key);
    if (it != g_shapes.end()) return it->second;
    ShapeInfo s{};
    for (int shift = 2; shift >= 1; --shift) {
        s.side_wg = shift == 2 ? SIDE_WG_QUARTER : SIDE_WG;
        s.plan = build_plan(M, N, shift);
        s.band[1] = band_flops(s.plan, BAKRON_ORDER_LA_FIRST, M, N);
        s.band[2] = band_flops(s.plan, BAKRON_ORDER_LB_FIRST, M, N);
        s.auto_order = s.band[2].exec < s.band[1].exec ? BAKRON_ORDER_LB_FIRST : BAKRON_ORDER_LA_FIRST;
        if (s.band[s.auto_order].side_useful <= SIDE_BUDGET * (M + N - 1)) break;
    }
    pull_counts(M, N, &s.pull_flops, &s.pull_leaves);
    s.side_ops = 0;
    for (const Op &op : s.plan.ops) s.side_ops += op.kind == OP_BAND && op.side;
    return g_shapes.emplace(key, s).first->second;
}

thread_local bool g_phase_valid = false;
thread_local double g_phase_ms[10];

struct Buffers {
    float *Wp, *Ebuf, *Tbuf, *LAp, *LBp, *sc, *zp, *Cd, *Cr;
    double *partial;
    int *ctr;  // tile counters of the deferred products
    int nctr;
    float4 *tabA;  // the leaf's LA band table, np x 2 float4 (tables_kernel)
    float *tabI, *ilb;
};

// T has one mp x np slab per buffer of the plan (of the whole grid, or of the
// parts of a split solve).
size_t carve(void *ws, int64_t mp, int64_t np, Buffers *b) {
    Carver cv(ws);
    const int M = (int)(mp / TB), N = (int)(np / TB);
    int slabs = shape_info(M, N).plan.slabs;
    if (N >= 2) slabs = std::max({slabs, shape_info(M, N / 2).plan.slabs, shape_info(M, N - N / 2).plan.slabs});
    if (M >= 2) slabs = std::max({slabs, shape_info(M / 2, N).plan.slabs, shape_info(M - M / 2, N).plan.slabs});
    float *Wp = cv.take<float>(mp * np);
    float *Eb = cv.take<float>(mp * np);
    float *Tb = cv.take<float>(mp * np * slabs);
    float *LAp = cv.take<float>(np * np);
    float *LBp = cv.take<float>(mp * mp);
    float *sc = cv.take<float>(mp);
    float *zp = cv.take<float>(mp);
    double *part = cv.take<double>(NPART);
    float *Cd = cv.take<float>(mp * np);
    float *Cr = cv.take<float>(mp * np);
    // counters for the plan of the whole grid and of the parts of a split solve
    int nctr = std::max(1, shape_info(M, N).side_ops);
    if (N >= 2) nctr = std::max({nctr, shape_info(M, N / 2).side_ops, shape_info(M, N - N / 2).side_ops});
    if (M >= 2) nctr = std::max({nctr, shape_info(M / 2, N).side_ops, shape_info(M - M / 2, N).side_ops});
    int *ctr = cv.take<int>(nctr * SIDE_QUEUES);
    float4 *tabA = cv.take<float4>(2 * np);
    float *tabI = cv.take<float>(np);
    float *ilb = cv.take<float>(mp);
    if (b) *b = Buffers{Wp, Eb, Tb, LAp, LBp, sc, zp, Cd, Cr, part, ctr, nctr * SIDE_QUEUES, tabA, tabI, ilb};
    return cv.used;
}

bool valid_quantizer(int32_t kind, int32_t bits) {
    if (kind == BAKRON_Q_SYM) return bits == 2 || bits == 3 || bits == 4 || bits == 8;
    if (kind == BAKRON_Q_ASYM) return bits == 2 || bits == 3 || bits == 4;
    return kind == BAKRON_Q_UNIT;
}

constexpr int64_t MAX_DIM = int64_t(1) << 20;

}  // namespace
}  // namespace bakron

using namespace bakron;

extern "C" size_t bakron_quantize_workspace_size(int64_t m, int64_t n, int32_t qkind, int32_t qbits) {
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM || !valid_quantizer(qkind, qbits)) return 0;
    char *base = reinterpret_cast<char *>(256);  // any aligned address: only sizes matter
    return carve(base, round_up(m, TB), round_up(n, TB), nullptr);
}

extern "C" int32_t bakron_schedule_info(int64_t m, int64_t n, int32_t flags, double *out) {
    clear_error();
    BK_REQUIRE(out != nullptr, "out is NULL");
    BK_REQUIRE(m >= 1 && n >= 1 && m <= MAX_DIM && n <= MAX_DIM, "bad shape %lld x %lld",
               (long long)m, (long long)n);
    const int M = (int)(round_up(m, TB) / TB), N = (int)(round_up(n, TB) / TB);
    const ShapeInfo &si = shape_info(M, N);
    int order = flags & BAKRON_ORDER_MASK;
    if (order == BAKRON_ORDER_AUTO || order == 3) order = si.auto_order;
    const int D = M + N - 1;
    out[0] = TB;
    out[1] = D;
    out[2] = si.band[order].launches;
    out[3] = (double)D * (2 * TB - 1);
    out[4] = order;
    out[5] = algorithmic_band_flops(m, n);
    out[6] = si.band[order].exec;
    out[7] = (double)m * (double)n * (double)(m + n);
    out[8] = (double)M * N * TB * TB * 4.0 * TB;
    out[9] = depth_of(D);
    out[10] = si.band[order].useful;
    out[11] = si.pull_flops;
    out[12] = si.pull_leaves;
    out[13] = si.band[order].side_launches;
    out[14] = si.band[order].side_useful;
    return BAKRON_OK;
}

extern "C" int32_t bakron_schedule_plan(int64_t m, int64_t n, int32_t flags, int32_t *ops,
                                        int64_t cap, int64_t *count) {
    clear_error();
    BK_REQUIRE(count != nullptr, "count is NULL");
    BK_REQUIRE(m >= 1 && n >= 1 && m <= MAX_DIM && n <= MAX_DIM, "bad shape %lld x %lld",
               (long long)m, (long long)n);
    const int M = (int)(round_up(m, TB) / TB), N = (int)(round_up(n, TB) / TB);
    const ShapeInfo &si = shape_info(M, N);
    int order = flags & BAKRON_ORDER_MASK;
    if (order == BAKRON_ORDER_AUTO || order == 3) order = si.auto_order;
    *count = (int64_t)si.plan.ops.size();
    BK_REQUIRE(ops == nullptr || cap >= *count, "ops holds %lld entries, the plan has %lld",
               (long long)cap, (long long)*count);
    if (!ops) return BAKRON_OK;
    for (size_t k = 0; k < si.plan.ops.size(); ++k) {
        const Op &op = si.plan.ops[k];
        int32_t *o = ops + 16 * k;
        for (int f = 0; f < 16; ++f) o[f] = -1;
        o[0] = op.kind;
        o[1] = op.side;
        o[2] = op.ev;
        if (op.kind == OP_LEAF) {
            o[3] = op.nd.K;
            o[4] = op.nd.flags;
        } else if (op.kind == OP_BAND) {
            o[3] = op.nd.K; o[5] = op.nd.L; o[6] = op.nd.H; o[7] = op.nd.slab;
            o[8] = op.prod; o[9] = op.lo; o[10] = op.hi;
            int mode, olo, cols, rlo, rows;
            if (band_geometry(op, order, M, N, mode, olo, cols, rlo, rows)) {
                o[11] = mode; o[12] = olo; o[13] = cols; o[14] = rlo; o[15] = rows;
            }
        }
    }
    return BAKRON_OK;
}

extern "C" int32_t bakron_last_phase_ms(double *out) {
    clear_error();
    BK_REQUIRE(out != nullptr, "out is NULL");
    BK_REQUIRE(g_phase_valid, "no timed bakron_quantize call on this thread");
    for (int k = 0; k < 10; ++k) out[k] = g_phase_ms[k];
    return BAKRON_OK;
}

namespace bakron {
namespace {

// Everything one solve enqueues, given validated arguments.
struct Solve {
    const float *W, *LA, *LB;
    int64_t m, n, mp, np;
    int M, N, order, qkind, qbits, qmin, qmax;
    int mse;    // per-row scale shrink by MSE search
    int split;  // SPLIT_NONE, SPLIT_COLS, SPLIT_ROWS: the hybrid schedule's top-level split
    int8_t *codes;
    float *scales, *zeros, *V, *E;
    int64_t ldo;  // row stride of codes, V, E (the full n; a part's m, n are its bounds)
    double *sum_e2;
    int32_t *dev_status;
    Buffers b;
};

// The hybrid schedule (BaKron-recursive's row / column split at the top level,
// Algorithm 6 below; pith.science review of arXiv 2608.06291, "Circularity
// Check": the recurrence F(m,n) - F(m,n1) - F(m,n2) = 2 m n1 n2 of Appendix C).
// A column split at tile J1 solves the columns 0 .. J1-1, applies their
// updates to the rest, W2 -= LB E1 LA21^T, then solves the columns J1 ..; a
// row split at I1 likewise with W2 -= LB21 E1 LA^T.  Both visit the entries
// in an order that extends the product order, so the result is the same
// (Theorem 3.2, "Core claim").
constexpr int SPLIT_NONE = 0, SPLIT_COLS = 1, SPLIT_ROWS = 2;

// The tile block rows I0 .. I0+Ms-1, columns J0 .. J0+Ns-1 of a solve, as a
// solve of its own over the same buffers (pointers moved to the block, strides
// kept).
Solve part_view(const Solve &sv, int I0, int J0, int Ms, int Ns) {
    Solve p = sv;
    const int64_t r0 = (int64_t)I0 * TB, c0 = (int64_t)J0 * TB;
    p.M = Ms;
    p.N = Ns;
    p.m = std::min<int64_t>(sv.m - r0, (int64_t)Ms * TB);
    p.n = std::min<int64_t>(sv.n - c0, (int64_t)Ns * TB);
    p.b.Wp += r0 * sv.np + c0;
    p.b.Cd += r0 * sv.np + c0;
    p.b.Cr += r0 * sv.np + c0;
    p.b.LAp += c0 * sv.np + c0;
    p.b.LBp += r0 * sv.mp + r0;
    p.b.sc += r0;
    p.b.zp += r0;
    p.b.tabA += 2 * c0;
    p.b.tabI += c0;
    p.b.ilb += r0;
    p.b.Ebuf += sv.order == BAKRON_ORDER_LA_FIRST ? r0 * sv.np + c0 : c0 * sv.mp + r0;
    p.codes += r0 * sv.ldo + c0;
    if (p.V) p.V += r0 * sv.ldo + c0;
    if (p.E) p.E += r0 * sv.ldo + c0;
    return p;
}

// the parts of a solve: (I0, J0, M, N) of each, in the order they run
int solve_parts(const Solve &sv, int part[2][4]) {
    if (sv.split == SPLIT_COLS) {
        const int J1 = sv.N / 2;
        part[0][0] = 0; part[0][1] = 0; part[0][2] = sv.M; part[0][3] = J1;
        part[1][0] = 0; part[1][1] = J1; part[1][2] = sv.M; part[1][3] = sv.N - J1;
        return 2;
    }
    if (sv.split == SPLIT_ROWS) {
        const int I1 = sv.M / 2;
        part[0][0] = 0; part[0][1] = 0; part[0][2] = I1; part[0][3] = sv.N;
        part[1][0] = I1; part[1][1] = 0; part[1][2] = sv.M - I1; part[1][3] = sv.N;
        return 2;
    }
    part[0][0] = 0; part[0][1] = 0; part[0][2] = sv.M; part[0][3] = sv.N;
    return 1;
}

// events a solve's plans need (its parts run one after the other)
int solve_events(const Solve &sv) {
    int part[2][4], ev = 0;
    const int np_ = solve_parts(sv, part);
    for (int k = 0; k < np_; ++k) ev = std::max(ev, shape_info(part[k][2], part[k][3]).plan.events);
    return ev + 2;  // and the set-up's fork and join
}

int32_t launch_band(const Solve &sv, const Op &op, int *ctr, hipStream_t stream, int *launched);

// One dense product of a split solve's cross update (band_gemm_kernel mode 4):
// C (rows x cols tiles) =|-= A B^T over kt K blocks, cut at the row (tri 1:
// A lower triangular) or the column (tri 2: B lower triangular).
int32_t launch_dense(const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
                     int64_t ldc, int rows, int cols, int kt, int tri, int subtract,
                     hipStream_t stream) {
    if (rows <= 0 || cols <= 0 || kt <= 0) return BAKRON_OK;
    BandArgs g{A, B, C, lda, ldb, ldc, 4, 0, kt, tri, rows, cols, 0, subtract, rows, 0, cols};
    hipLaunchKernelGGL(band_gemm_kernel, dim3(cols, (rows + 7) & ~7), dim3(256), 0, stream, g);
    BK_LAUNCH_CHECK("band_gemm_kernel");
    return BAKRON_OK;
}

// The cross update of a split solve, between its parts: the first part's E
// applied to the second part's W (the part at tile row I1 or column J1; T of
// depth 0 holds the intermediate product).
int32_t cross_update(const Solve &sv, int I1, int J1, hipStream_t stream) {
    const Buffers &b = sv.b;
    const int64_t mp = sv.mp, np = sv.np, r1 = (int64_t)I1 * TB, c1 = (int64_t)J1 * TB;
    const int M = sv.M, N = sv.N;
    float *T = b.Tbuf;
    const bool la_first = sv.order == BAKRON_ORDER_LA_FIRST;
    int32_t st;
    if (sv.split == SPLIT_COLS) {  // W2 -= LB E1 LA21^T
        if (la_first) {            // Tt(J', I) = sum_J LA21(J', J) E(I, J); W2 -= LB Tt^T
            st = launch_dense(b.LAp + c1 * np, np, b.Ebuf, np, T, mp, N - J1, M, J1, 0, BW_STORE, stream);
            if (st == BAKRON_OK)
                st = launch_dense(b.LBp, mp, T, mp, b.Wp + c1, np, M, N - J1, M, 1, BW_SUB, stream);
        } else {                   // S(I', J) = sum_I LB(I', I) E(I, J); W2 -= S LA21^T
            st = launch_dense(b.LBp, mp, b.Ebuf, mp, T, np, M, J1, M, 1, BW_STORE, stream);
            if (st == BAKRON_OK)
                st = launch_dense(T, np, b.LAp + c1 * np, np, b.Wp + c1, np, M, N - J1, J1, 0, BW_SUB, stream);
        }
    } else {                       // W2 -= LB21 E1 LA^T
        if (la_first) {            // Tt(J', I) = sum_J LA(J', J) E(I, J), I < I1; W2 -= LB21 Tt^T
            st = launch_dense(b.LAp, np, b.Ebuf, np, T, mp, N, I1, N, 1, BW_STORE, stream);
            if (st == BAKRON_OK)
                st = launch_dense(b.LBp + r1 * mp, mp, T, mp, b.Wp + r1 * np, np, M - I1, N, I1, 0, BW_SUB, stream);
        } else {                   // S(I', J) = sum_{I < I1} LB21(I', I) E(I, J); W2 -= S LA^T
            st = launch_dense(b.LBp + r1 * mp, mp, b.Ebuf, mp, T, np, M - I1, N, I1, 0, BW_STORE, stream);
            if (st == BAKRON_OK)
                st = launch_dense(T, np, b.LAp, np, b.Wp + r1 * np, np, M - I1, N, N, 2, BW_SUB, stream);
        }
    }
    return st;
}

// Enqueues the whole solve.  With `side` (and `sync`, the plan's events),
// deferred band products run on `side`, forked from and joined into `stream`;
// without, the plan runs in order on `stream`.  With `evs`, records an event
// after each step (-1 start, 0 prep, 1 leaf, 2 band product, 3 finalise,
// 4 deferred band product).
int32_t enqueue_solve(const Solve &sv, hipStream_t stream, hipStream_t side,
                      const std::vector<hipEvent_t> *sync, std::vector<hipEvent_t> *evs,
                      std::vector<int> *ev_phase) {
    auto mark = [&](int phase) -> int32_t {
        if (!evs) return BAKRON_OK;
        hipEvent_t e;
        BK_HIP_CHECK(hipEventCreate(&e));
        evs->push_back(e);
        ev_phase->push_back(phase);
        BK_HIP_CHECK(hipEventRecord(e, stream));
        return BAKRON_OK;
    };
#define BK_MARK(p)                    \
    do {                              \
        int32_t s_ = mark(p);         \
        if (s_ != BAKRON_OK) return s_; \
    } while (0)
    const Buffers &b = sv.b;
    const int64_t m = sv.m, n = sv.n, mp = sv.mp, np = sv.np;
    BK_MARK(-1);
    // the parts (one without a split) and, between them, the cross update
    int part[2][4];
    const int nparts = solve_parts(sv, part);
    // Set-up: row parameters and W's working copy, the factor copies, the leaf
    // tables.  With a side stream (one part), the critical stream prepares tile
    // rows and columns 0 .. PREP_TILES-1 and the side stream the rest, joined
    // before the first step that reaches past them: a leaf of diagonal >=
    // PREP_TILES-1 (a pushing leaf reads factor blocks one past its diagonal)
    // or a band node whose diagonals reach PREP_TILES.
    const bool split_prep = side && nparts == 1 && sv.M + sv.N - 1 > 2 * PREP_TILES;
    const int64_t rw = split_prep ? std::min<int64_t>(mp, (int64_t)PREP_TILES * TB) : mp;
    const int64_t ra = split_prep ? std::min<int64_t>(np, (int64_t)PREP_TILES * TB) : np;
    const int pe = split_prep ? solve_events(sv) - 2 : -1;
    if (split_prep) {
        BK_HIP_CHECK(hipEventRecord((*sync)[pe], stream));
        BK_HIP_CHECK(hipStreamWaitEvent(side, (*sync)[pe], 0));
    }
    const int w_vec = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(sv.W) & 15) == 0);
    const int a_vec = (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(sv.LA) & 15) == 0);
    const int b_vec = (m % 4 == 0) && ((reinterpret_cast<uintptr_t>(sv.LB) & 15) == 0);
    const unsigned rl_blocks = 256u * 8u;
    auto prep = [&](hipStream_t st, int64_t w0, int64_t w1, int64_t a0, int64_t a1, int clear) {
        if (w1 > w0)
            hipLaunchKernelGGL(qparams_kernel, dim3((unsigned)(w1 - w0)), dim3(256), 0, st, sv.W, m, n,
                               sv.qkind, sv.qbits, sv.scales, sv.zeros, b.sc, b.zp, sv.dev_status,
                               sv.mse, w_vec, b.Wp, np, w0);
        if (a1 > a0)
            hipLaunchKernelGGL(relayout_kernel, dim3(rl_blocks), dim3(256), 0, st, sv.LA, n, n, b.LAp,
                               np, np, 2, a_vec, a0, a1);
        if (w1 > w0)
            hipLaunchKernelGGL(relayout_kernel, dim3(rl_blocks), dim3(256), 0, st, sv.LB, m, m, b.LBp,
                               mp, mp, 2, b_vec, w0, w1);
        const int64_t span = std::max(a1 - a0, w1 - w0);
        hipLaunchKernelGGL(tables_kernel, dim3((unsigned)std::max<int64_t>(1, (span + 255) / 256)),
                           dim3(256), 0, st, b.LAp, b.LBp, np, mp, b.tabA, b.tabI, b.ilb, b.ctr,
                           clear ? b.nctr : 0, a0, a1, w0, w1);
    };
    prep(stream, 0, rw, 0, ra, 1);
    BK_LAUNCH_CHECK("set-up kernels");
    if (split_prep) {
        prep(side, rw, mp, ra, np, 0);
        BK_LAUNCH_CHECK("set-up kernels (side stream)");
        BK_HIP_CHECK(hipEventRecord((*sync)[pe + 1], side));
    }
    bool prep_joined = !split_prep;
    BK_MARK(0);

    const auto aligned = [](const void *p, uintptr_t to) {
        return (reinterpret_cast<uintptr_t>(p) & (to - 1)) == 0;
    };
    for (int k = 0; k < nparts; ++k) {
        if (k == 1) {
            const int32_t st = cross_update(sv, part[1][0], part[1][1], stream);
            if (st != BAKRON_OK) return st;
            BK_MARK(2);
        }
        const Solve pv = part_view(sv, part[k][0], part[k][1], part[k][2], part[k][3]);
        const Buffers &pb = pv.b;
        const int PM = pv.M, PN = pv.N;
        const int out_vec = sv.ldo % 4 == 0 && aligned(pv.codes, 4) && aligned(pv.V, 16) &&
                            aligned(pv.E, 16);
        LeafArgs la{pb.Wp, pb.Ebuf, pb.LAp, pb.LBp, pb.sc, pb.zp, mp, np, PM, PN, sv.order,
                    sv.qmin, sv.qmax, pv.codes, pv.V, pv.E, pv.m, pv.n, sv.dev_status, pb.Cd, pb.Cr,
                    out_vec, sv.ldo, pb.tabA, pb.tabI, pb.ilb};
        const Plan &plan = shape_info(PM, PN).plan;
        if (k > 0) {  // the first part's counters were cleared by tables_kernel
            hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(256), 0, stream, b.ctr, b.nctr);
            BK_LAUNCH_CHECK("zero_i32_kernel");
        }
        int side_k = 0;
        for (const Op &op : plan.ops) {
            if (op.kind == OP_RECORD || op.kind == OP_WAIT) {
                if (!side) continue;
                hipStream_t st = op.side ? side : stream;
                if (op.kind == OP_RECORD) BK_HIP_CHECK(hipEventRecord((*sync)[op.ev], st));
                else BK_HIP_CHECK(hipStreamWaitEvent(st, (*sync)[op.ev], 0));
                continue;
            }
            const Node &nd = op.nd;
            const bool crit = op.kind == OP_LEAF || !op.side || !side;
            if (!prep_joined && crit &&
                (op.kind == OP_LEAF ? nd.K >= PREP_TILES - 1 : nd.K + nd.L > PREP_TILES)) {
                BK_HIP_CHECK(hipStreamWaitEvent(stream, (*sync)[pe + 1], 0));
                prep_joined = true;
            }
            if (op.kind == OP_LEAF) {
                const int Ilo = std::max(0, nd.K - PN + 1), Ihi = std::min(PM - 1, nd.K);
                const unsigned nwg = (unsigned)(Ihi - Ilo + 1);
                if (sv.qkind == BAKRON_Q_ASYM)
                    hipLaunchKernelGGL(leaf_kernel<true>, dim3(nwg), dim3(LEAF_THREADS), 0,
                                       stream, la, nd.K, nd.flags);
                else
                    hipLaunchKernelGGL(leaf_kernel<false>, dim3(nwg), dim3(LEAF_THREADS), 0,
                                       stream, la, nd.K, nd.flags);
                BK_LAUNCH_CHECK("leaf_kernel");
                BK_MARK(1);
                continue;
            }
            int *ctr = op.side ? b.ctr + SIDE_QUEUES * side_k++ : nullptr;
            int launched = 0;
            const int32_t st = launch_band(pv, op, ctr, op.side && side ? side : stream, &launched);
            if (st != BAKRON_OK) return st;
            if (launched) BK_MARK(op.side ? 4 : 2);
        }
    }
    if (!prep_joined) BK_HIP_CHECK(hipStreamWaitEvent(stream, (*sync)[pe + 1], 0));
    if (sv.sum_e2) {
        hipLaunchKernelGGL(sumsq_partial_kernel, dim3(NPART), dim3(256), 0, stream, b.Ebuf,
                           mp * np, b.partial);
        hipLaunchKernelGGL(sumsq_final_kernel, dim3(1), dim3(256), 0, stream, b.partial, sv.sum_e2);
        BK_LAUNCH_CHECK("sumsq kernels");
    }
    BK_MARK(3);
#undef BK_MARK
    return BAKRON_OK;
}

// Executable graphs of whole solves, keyed by every argument the kernels bake
// in (device, pointers, sizes, quantizer, product order).  A replay reads the
// buffers' current contents.  At most kGraphCache entries; the least recently
// used one is dropped.
struct GraphKey {
    int dev, order, qkind, qbits, mse, split;
    int64_t m, n;
    const void *p[12];
    bool operator<(const GraphKey &o) const {
        if (dev != o.dev) return dev < o.dev;
        if (order != o.order) return order < o.order;
        if (qkind != o.qkind) return qkind < o.qkind;
        if (qbits != o.qbits) return qbits < o.qbits;
        if (mse != o.mse) return mse < o.mse;
        if (split != o.split) return split < o.split;
        if (m != o.m) return m < o.m;
        if (n != o.n) return n < o.n;
        for (int k = 0; k < 12; ++k)
            if (p[k] != o.p[k]) return p[k] < o.p[k];
        return false;
    }
};

struct GraphEntry {
    hipGraphExec_t exec;
    hipEvent_t done;  // recorded on the launch stream after every launch
    uint64_t last_use;
};

constexpr size_t kGraphCache = 16;
std::mutex g_graph_mu;
std::map<GraphKey, GraphEntry> g_graphs;
uint64_t g_graph_clock = 0;

// Per device: the streams a graph is captured on, the side stream of eager
// solves, and the plan's fork / join events (one set for captures, one for
// eager solves; each set is used under its own lock).
struct DevStreams {
    hipStream_t cap = nullptr, cap_side = nullptr, side = nullptr;
    std::vector<hipEvent_t> cap_ev, ev;
};
std::map<int, DevStreams> g_dev;
std::mutex g_eager_mu;

int32_t grow_events(std::vector<hipEvent_t> &v, int n) {
    while ((int)v.size() < n) {
        hipEvent_t e;
        BK_HIP_CHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
        v.push_back(e);
    }
    return BAKRON_OK;
}

int32_t make_stream(hipStream_t *s) {
    if (!*s) BK_HIP_CHECK(hipStreamCreateWithFlags(s, hipStreamNonBlocking));
    return BAKRON_OK;
}

// Finds or builds the graph for `sv` and launches it on `stream`.  Lookup,
// capture, eviction and launch all happen under g_graph_mu, so no thread can
// destroy an executable graph between another thread's lookup and launch; an
// evicted graph is destroyed only after its last launch has completed.
int32_t launch_graph(const Solve &sv, int dev, const void *ws, hipStream_t stream) {
    GraphKey key{dev, sv.order, sv.qkind, sv.qbits, sv.mse, sv.split, sv.m, sv.n,
                 {sv.W, sv.LA, sv.LB, sv.codes, sv.scales, sv.zeros, sv.V, sv.E, sv.sum_e2,
                  sv.dev_status, ws, nullptr}};
    std::lock_guard<std::mutex> lock(g_graph_mu);
    auto it = g_graphs.find(key);
    if (it == g_graphs.end()) {
        DevStreams &ds = g_dev[dev];
        int32_t st = make_stream(&ds.cap);
        if (st == BAKRON_OK) st = make_stream(&ds.cap_side);
        if (st == BAKRON_OK) st = grow_events(ds.cap_ev, solve_events(sv));
        if (st != BAKRON_OK) return st;
        hipStream_t cs = ds.cap;
        BK_HIP_CHECK(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
        st = enqueue_solve(sv, cs, ds.cap_side, &ds.cap_ev, nullptr, nullptr);
        hipGraph_t graph = nullptr;
        hipError_t ce = hipStreamEndCapture(cs, &graph);
        if (st != BAKRON_OK) {
            if (graph) (void)hipGraphDestroy(graph);
            return st;
        }
        if (ce != hipSuccess) {
            set_error("hipStreamEndCapture: %s", hipGetErrorString(ce));
            return BAKRON_ERR_HIP;
        }
        hipGraphExec_t ge;
        hipError_t ie = hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0);
        (void)hipGraphDestroy(graph);
        if (ie != hipSuccess) {
            set_error("hipGraphInstantiate: %s", hipGetErrorString(ie));
            return BAKRON_ERR_HIP;
        }
        hipEvent_t done;
        ie = hipEventCreateWithFlags(&done, hipEventDisableTiming);
        if (ie != hipSuccess) {
            (void)hipGraphExecDestroy(ge);
            set_error("hipEventCreateWithFlags: %s", hipGetErrorString(ie));
            return BAKRON_ERR_HIP;
        }
        if (g_graphs.size() >= kGraphCache) {
            auto victim = g_graphs.begin();
            for (auto jt = g_graphs.begin(); jt != g_graphs.end(); ++jt)
                if (jt->second.last_use < victim->second.last_use) victim = jt;
            (void)hipEventSynchronize(victim->second.done);
            (void)hipGraphExecDestroy(victim->second.exec);
            (void)hipEventDestroy(victim->second.done);
            g_graphs.erase(victim);
        }
        it = g_graphs.emplace(key, GraphEntry{ge, done, 0}).first;
    }
    it->second.last_use = ++g_graph_clock;
    BK_HIP_CHECK(hipGraphLaunch(it->second.exec, stream));
    BK_HIP_CHECK(hipEventRecord(it->second.done, stream));
    return BAKRON_OK;
}

// Launches one band op of the plan (nothing when its range holds no tile).
int32_t launch_band(const Solve &sv, const Op &op, int *ctr, hipStream_t stream, int *launched) {
    const Buffers &b = sv.b;
    const Node &nd = op.nd;
    const int M = sv.M, N = sv.N;
    const int64_t mp = sv.mp, np = sv.np;
    int mode, olo, cols, rlo, rows;
    *launched = 0;
    if (!band_geometry(op, sv.order, M, N, mode, olo, cols, rlo, rows)) return BAKRON_OK;
    float *T = b.Tbuf + (int64_t)nd.slab * mp * np;
    BandArgs g{};
    switch (mode) {
    case 0: g = BandArgs{b.LAp, b.Ebuf, T, np, np, mp, 0, nd.K, nd.L, nd.H, M, N, rlo, 0, rows, olo, cols}; break;
    case 1: g = BandArgs{b.LBp, T, b.Wp, mp, mp, np, 1, nd.K, nd.L, nd.H, M, N, rlo, 1, rows, olo, cols}; break;
    case 2: g = BandArgs{b.LBp, b.Ebuf, T, mp, mp, np, 2, nd.K, nd.L, nd.H, M, N, rlo, 0, rows, olo, cols}; break;
    default: g = BandArgs{T, b.LAp, b.Wp, np, np, np, 3, nd.K, nd.L, nd.H, M, N, rlo, 1, rows, olo, cols}; break;
    }
    if (op.side) {
        // one workgroup per CU, up to one per tile
        const int wgs = std::min(shape_info(sv.M, sv.N).side_wg, cols * rows);
        hipLaunchKernelGGL(band_side_kernel, dim3(wgs), dim3(SIDE_THREADS), 0, stream, g, ctr,
                           sv.dev_status);
        BK_LAUNCH_CHECK("band_side_kernel");
    } else {
        hipLaunchKernelGGL(band_gemm_kernel, dim3(cols, (rows + 7) & ~7), dim3(256), 0, stream, g);
        BK_LAUNCH_CHECK("band_gemm_kernel");
    }
    *launched = 1;
    return BAKRON_OK;
}

// Time the plan's critical (side = 0) or deferred (side = 1) band launches on
// their own: they are captured in plan order into a one-off graph, which
// dispatches each as soon as the previous one ends, and the graph launch is
// bracketed by two events on `stream`.  They rewrite the workspace's W and T
// from its current contents (the solve's outputs are not touched); the counters
// of the deferred launches are cleared first.  Returns the elapsed ms.
int32_t replay_band(const Solve &sv, int dev, hipStream_t stream, int side, double *ms_out) {
    const Plan &plan = shape_info(sv.M, sv.N).plan;
    hipGraphExec_t ge = nullptr;
    int32_t st = BAKRON_OK;
    {
        std::lock_guard<std::mutex> lock(g_graph_mu);
        DevStreams &ds = g_dev[dev];
        st = make_stream(&ds.cap);
        if (st != BAKRON_OK) return st;
        BK_HIP_CHECK(hipStreamBeginCapture(ds.cap, hipStreamCaptureModeThreadLocal));
        if (side) hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(256), 0, ds.cap, sv.b.ctr, sv.b.nctr);
        int side_k = 0;
        for (const Op &op : plan.ops) {
            if (op.kind != OP_BAND) continue;
            int *ctr = op.side ? sv.b.ctr + SIDE_QUEUES * side_k++ : nullptr;
            if (op.side != side) continue;
            int launched = 0;
            st = launch_band(sv, op, ctr, ds.cap, &launched);
            if (st != BAKRON_OK) break;
        }
        hipGraph_t graph = nullptr;
        const hipError_t ce = hipStreamEndCapture(ds.cap, &graph);
        if (st == BAKRON_OK && ce != hipSuccess) {
            set_error("hipStreamEndCapture: %s", hipGetErrorString(ce));
            st = BAKRON_ERR_HIP;
        }
        if (st == BAKRON_OK) {
            const hipError_t ie = hipGraphInstantiate(&ge, graph, nullptr, nullptr, 0);
            if (ie != hipSuccess) {
                set_error("hipGraphInstantiate: %s", hipGetErrorString(ie));
                st = BAKRON_ERR_HIP;
            }
        }
        if (graph) (void)hipGraphDestroy(graph);
    }
    if (st != BAKRON_OK) return st;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = hipEventRecord(e0, stream);
    if (e == hipSuccess) e = hipGraphLaunch(ge, stream);
    if (e == hipSuccess) e = hipEventRecord(e1, stream);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess) {
        set_error("band replay: %s", hipGetErrorString(e));
        st = BAKRON_ERR_HIP;
    }
    *ms_out = ms;
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipGraphExecDestroy(ge);
    return st;
}

}  // namespace
}  // namespace bakron

namespace bakron {
namespace {

// Argument checks shared by bakron_quantize and bakron_quantize_noalloc, then
// the solve's description (without its workspace buffers).
int32_t make_solve(const float *W, int64_t m, int64_t n, const float *LA, const float *LB,
                   int32_t qkind, int32_t qbits, int8_t *codes, float *scales, float *zeros,
                   float *V, float *E, double *sum_e2, int32_t *dev_status, int32_t flags,
                   Solve *out) {
    BK_REQUIRE(W && LA && LB && codes && scales, "W, LA, LB, codes and scales must be non-NULL");
    BK_REQUIRE(m >= 1 && n >= 1 && m <= MAX_DIM && n <= MAX_DIM, "bad shape %lld x %lld",
               (long long)m, (long long)n);
    BK_REQUIRE(valid_quantizer(qkind, qbits), "unsupported quantizer kind=%d bits=%d", qkind, qbits);
    BK_REQUIRE((flags & ~(BAKRON_ORDER_MASK | BAKRON_FLAG_PHASE_TIMING | BAKRON_FLAG_NO_GRAPH |
                          BAKRON_FLAG_MSE_SCALE | BAKRON_FLAG_SPLIT_COLS | BAKRON_FLAG_SPLIT_ROWS)) == 0 &&
                   (flags & BAKRON_ORDER_MASK) != 3,
               "unknown flags 0x%x", flags);
    BK_REQUIRE(!((flags & BAKRON_FLAG_SPLIT_COLS) && (flags & BAKRON_FLAG_SPLIT_ROWS)),
               "BAKRON_FLAG_SPLIT_COLS and BAKRON_FLAG_SPLIT_ROWS exclude each other");
    BK_REQUIRE(!((flags & (BAKRON_FLAG_SPLIT_COLS | BAKRON_FLAG_SPLIT_ROWS)) &&
                 (flags & BAKRON_FLAG_PHASE_TIMING)),
               "BAKRON_FLAG_PHASE_TIMING times the unsplit schedule only (no BAKRON_FLAG_SPLIT_*)");
    Solve sv{};
    sv.W = W; sv.LA = LA; sv.LB = LB; sv.m = m; sv.n = n;
    sv.mp = round_up(m, TB);
    sv.np = round_up(n, TB);
    sv.M = (int)(sv.mp / TB);
    sv.N = (int)(sv.np / TB);
    const ShapeInfo &si = shape_info(sv.M, sv.N);
    sv.order = flags & BAKRON_ORDER_MASK;
    if (sv.order == BAKRON_ORDER_AUTO) sv.order = si.auto_order;
    sv.qkind = qkind;
    sv.qbits = qbits;
    sv.mse = (flags & BAKRON_FLAG_MSE_SCALE) && qkind != BAKRON_Q_UNIT;
    if (qkind == BAKRON_Q_SYM) { sv.qmin = -(1 << (qbits - 1)); sv.qmax = (1 << (qbits - 1)) - 1; }
    else if (qkind == BAKRON_Q_ASYM) { sv.qmin = 0; sv.qmax = (1 << qbits) - 1; }
    else { sv.qmin = -128; sv.qmax = 127; }
    sv.codes = codes; sv.scales = scales; sv.zeros = zeros; sv.V = V; sv.E = E;
    sv.ldo = n;
    sv.sum_e2 = sum_e2; sv.dev_status = dev_status;
    // a split of a one-tile dimension leaves nothing to split
    sv.split = (flags & BAKRON_FLAG_SPLIT_COLS) && sv.N >= 2   ? SPLIT_COLS
               : (flags & BAKRON_FLAG_SPLIT_ROWS) && sv.M >= 2 ? SPLIT_ROWS
                                                               : SPLIT_NONE;
    *out = sv;
    return BAKRON_OK;
}

}  // namespace
}  // namespace bakron

extern "C" int32_t bakron_quantize(const float *W, int64_t m, int64_t n, const float *LA,
                                   const float *LB, int32_t qkind, int32_t qbits, int8_t *codes,
                                   float *scales, float *zeros, float *V, float *E,
                                   double *sum_e2, int32_t *dev_status, int32_t flags, void *ws,
                                   size_t ws_bytes, void *stream_) {
    clear_error();
    Solve sv{};
    int32_t st = make_solve(W, m, n, LA, LB, qkind, qbits, codes, scales, zeros, V, E, sum_e2,
                            dev_status, flags, &sv);
    if (st != BAKRON_OK) return st;
    const size_t need = bakron_quantize_workspace_size(m, n, qkind, qbits);
    if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) {
        set_error("workspace needs %zu bytes at 256-byte alignment (got %zu at %p)", need,
                  ws_bytes, ws);
        return BAKRON_ERR_WORKSPACE;
    }
    st = check_device();
    if (st != BAKRON_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    carve(ws, sv.mp, sv.np, &sv.b);

    if (flags & BAKRON_FLAG_PHASE_TIMING) {
        std::vector<hipEvent_t> evs;
        std::vector<int> ev_phase;
        st = enqueue_solve(sv, stream, nullptr, nullptr, &evs, &ev_phase);
        if (st == BAKRON_OK) {
            hipError_t e = hipEventSynchronize(evs.back());
            if (e != hipSuccess) {
                set_error("hipEventSynchronize: %s", hipGetErrorString(e));
                st = BAKRON_ERR_HIP;
            } else {
                for (int k = 0; k < 10; ++k) g_phase_ms[k] = 0.0;
                for (size_t k = 1; k < evs.size(); ++k) {
                    float ms = 0.0f;
                    (void)hipEventElapsedTime(&ms, evs[k - 1], evs[k]);
                    const int ph = ev_phase[k];
                    g_phase_ms[ph == 4 ? 6 : ph] += ms;
                    if (ph == 1) g_phase_ms[4] += 1;
                    if (ph == 2) g_phase_ms[5] += 1;
                    if (ph == 4) g_phase_ms[7] += 1;
                }
            }
        }
        for (hipEvent_t e : evs) (void)hipEventDestroy(e);
        int dev = 0;
        BK_HIP_CHECK(hipGetDevice(&dev));
        if (st == BAKRON_OK) st = replay_band(sv, dev, stream, 0, &g_phase_ms[8]);
        if (st == BAKRON_OK) st = replay_band(sv, dev, stream, 1, &g_phase_ms[9]);
        g_phase_valid = st == BAKRON_OK;
        return st;
    }
    int dev = 0;
    BK_HIP_CHECK(hipGetDevice(&dev));
    if (flags & BAKRON_FLAG_NO_GRAPH) {
        std::lock_guard<std::mutex> lock(g_eager_mu);
        DevStreams *ds;
        {
            std::lock_guard<std::mutex> glock(g_graph_mu);
            ds = &g_dev[dev];
        }
        st = make_stream(&ds->side);
        if (st == BAKRON_OK) st = grow_events(ds->ev, solve_events(sv));
        if (st != BAKRON_OK) return st;
        return enqueue_solve(sv, stream, ds->side, &ds->ev, nullptr, nullptr);
    }
    return launch_graph(sv, dev, ws, stream);
}

// --------------------------------------------------------------------------
// bakron_quantize_noalloc: the solve for callers that cannot allocate device
// memory.  Its workspace is `scratch`, a fixed array of device memory: each
// GPU the library runs on holds its own copy until the process ends.  In host
// code the name `scratch` denotes a host-side stand-in, not a device address;
// the device address of the current GPU's copy comes from
// hipGetSymbolAddress, taken once per device (that device current) on the
// entry point's first call there, and only that address reaches the kernels.
static __device__ __align__(256) unsigned char scratch[BAKRON_NOALLOC_SCRATCH_BYTES];

namespace bakron {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device

int32_t scratch_address(void **ptr) {
    int dev = 0;
    BK_HIP_CHECK(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device index %d out of range", dev);
        return BAKRON_ERR_UNSUPPORTED_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        BK_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255) != 0) {
            set_error("hipGetSymbolAddress(scratch) gave %p", p);
            return BAKRON_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return BAKRON_OK;
}

}  // namespace
}  // namespace bakron

extern "C" int32_t bakron_quantize_noalloc(const float *W, int64_t m, int64_t n, const float *LA,
                                           const float *LB, int32_t qkind, int32_t qbits,
                                           int8_t *codes, float *scales, float *zeros, float *V,
                                           float *E, double *sum_e2, int32_t *dev_status,
                                           int32_t flags, void *stream_) {
    clear_error();
    BK_REQUIRE(!(flags & BAKRON_FLAG_PHASE_TIMING),
               "BAKRON_FLAG_PHASE_TIMING creates events; bakron_quantize_noalloc does not take it");
    Solve sv{};
    int32_t st = make_solve(W, m, n, LA, LB, qkind, qbits, codes, scales, zeros, V, E, sum_e2,
                            dev_status, flags, &sv);
    if (st != BAKRON_OK) return st;
    const size_t need = bakron_quantize_workspace_size(m, n, qkind, qbits);
    if (need > BAKRON_NOALLOC_SCRATCH_BYTES) {
        set_error("a %lld x %lld solve needs %zu bytes of workspace; bakron_quantize_noalloc has "
                  "%zu (use bakron_quantize with a workspace)",
                  (long long)m, (long long)n, need, (size_t)BAKRON_NOALLOC_SCRATCH_BYTES);
        return BAKRON_ERR_WORKSPACE;
    }
    st = check_device();
    if (st != BAKRON_OK) return st;
    void *ptr = nullptr;
    st = scratch_address(&ptr);
    if (st != BAKRON_OK) return st;
    carve(ptr, sv.mp, sv.np, &sv.b);
    // the plan in order on the caller's stream: no side stream, event or graph
    return enqueue_solve(sv, static_cast<hipStream_t>(stream_), nullptr, nullptr, nullptr, nullptr);
}

// --------------------------------------------------------------------------
// BaKron-antidiagonal: one entry anti-diagonal at a time (comparison variant).
namespace bakron {
namespace {
size_t carve_antidiag(void *ws, int64_t m, int64_t n, float **Wp, float **LAp, float **LBp,
                      float **sc, float **zp, float **eb) {
    const int64_t mp = round_up(m, TB), np = round_up(n, TB);
    Carver cv(ws);
    float *w_ = cv.take<float>(mp * np);
    float *la = cv.take<float>(np * np);
    float *lb = cv.take<float>(mp * mp);
    float *s_ = cv.take<float>(mp);
    float *z_ = cv.take<float>(mp);
    float *e_ = cv.take<float>(std::min(m, n));
    if (Wp) { *Wp = w_; *LAp = la; *LBp = lb; *sc = s_; *zp = z_; *eb = e_; }
    return cv.used;
}
}  // namespace
}  // namespace bakron

extern "C" size_t bakron_quantize_antidiag_workspace_size(int64_t m, int64_t n, int32_t qkind,
                                                          int32_t qbits) {
    if (m < 1 || n < 1 || m > MAX_DIM || n > MAX_DIM || !valid_quantizer(qkind, qbits)) return 0;
    return carve_antidiag(reinterpret_cast<void *>(256), m, n, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr);
}

extern "C" int32_t bakron_quantize_antidiag(const float *W, int64_t m, int64_t n, const float *LA,
                                            const float *LB, int32_t qkind, int32_t qbits,
                                            int8_t *codes, float *scales, float *zeros, float *V,
                                            float *E, int32_t *dev_status, void *ws,
                                            size_t ws_bytes, void *stream_) {
    clear_error();
    BK_REQUIRE(W && LA && LB && codes && scales, "W, LA, LB, codes and scales must be non-NULL");
    BK_REQUIRE(m >= 1 && n >= 1 && m <= MAX_DIM && n <= MAX_DIM, "bad shape %lld x %lld",
               (long long)m, (long long)n);
    BK_REQUIRE(valid_quantizer(qkind, qbits), "unsupported quantizer kind=%d bits=%d", qkind, qbits);
    const size_t need = bakron_quantize_antidiag_workspace_size(m, n, qkind, qbits);
    if (ws == nullptr || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) {
        set_error("workspace needs %zu bytes at 256-byte alignment (got %zu at %p)", need,
                  ws_bytes, ws);
        return BAKRON_ERR_WORKSPACE;
    }
    int32_t st = check_device();
    if (st != BAKRON_OK) return st;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int64_t mp = round_up(m, TB), np = round_up(n, TB);
    const int M = (int)(mp / TB), N = (int)(np / TB);
    float *Wp, *LAp, *LBp, *sc, *zp, *eb;
    carve_antidiag(ws, m, n, &Wp, &LAp, &LBp, &sc, &zp, &eb);
    int qmin, qmax;
    if (qkind == BAKRON_Q_SYM) { qmin = -(1 << (qbits - 1)); qmax = (1 << (qbits - 1)) - 1; }
    else if (qkind == BAKRON_Q_ASYM) { qmin = 0; qmax = (1 << qbits) - 1; }
    else { qmin = -128; qmax = 127; }
    hipLaunchKernelGGL(qparams_kernel, dim3((unsigned)mp), dim3(256), 0, stream, W, m, n, qkind, qbits,
                       scales, zeros, sc, zp, dev_status, 0,
                       (int)((n % 4 == 0) && ((reinterpret_cast<uintptr_t>(W) & 15) == 0)), nullptr,
                       (int64_t)0, (int64_t)0);
    BK_LAUNCH_CHECK("qparams_kernel");
    const unsigned rl_blocks = 256u * 8u;
    hipLaunchKernelGGL(relayout_kernel, dim3(rl_blocks), dim3(256), 0, stream, W, m, n, Wp, mp, np, 0, 0,
                       (int64_t)0, mp);
    hipLaunchKernelGGL(relayout_kernel, dim3(rl_blocks), dim3(256), 0, stream, LA, n, n, LAp, np, np, 1, 0,
                       (int64_t)0, np);
    hipLaunchKernelGGL(relayout_kernel, dim3(rl_blocks), dim3(256), 0, stream, LB, m, m, LBp, mp, mp, 1, 0,
                       (int64_t)0, mp);
    BK_LAUNCH_CHECK("relayout_kernel");
    for (int d = 0; d <= (int)(m + n - 2); ++d) {
        const int i_min = (int)std::max<int64_t>(0, d - n + 1), i_max = (int)std::min<int64_t>(m - 1, d);
        const int cnt = i_max - i_min + 1;
        if (qkind == BAKRON_Q_ASYM)
            hipLaunchKernelGGL(ad_round_kernel<true>, dim3((cnt + 255) / 256), dim3(256), 0, stream, Wp, LAp,
                               LBp, sc, zp, mp, np, n, d, i_min, cnt, (float)qmin, (float)qmax, codes, V, E,
                               eb, dev_status);
        else
            hipLaunchKernelGGL(ad_round_kernel<false>, dim3((cnt + 255) / 256), dim3(256), 0, stream, Wp, LAp,
                               LBp, sc, zp, mp, np, n, d, i_min, cnt, (float)qmin, (float)qmax, codes, V, E,
                               eb, dev_status);
        BK_LAUNCH_CHECK("ad_round_kernel");
        if (d == (int)(m + n - 2)) break;
        const int ti0 = i_min / TB, tj0 = (d - i_max) / TB;
        hipLaunchKernelGGL(ad_update_kernel, dim3(N - tj0, M - ti0), dim3(256), 0, stream, Wp, LAp, LBp, eb,
                           mp, np, d, i_min, cnt, ti0, tj0);
        BK_LAUNCH_CHECK("ad_update_kernel");
    }
    return BAKRON_OK;
}
