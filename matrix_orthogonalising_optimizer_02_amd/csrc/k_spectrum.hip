// Singular-spectrum diagnostic: the SVD entropy of "Muon is Scalable for LLM Training",
// Sec. 3.4 (Dynamics of Singular Spectrum). For a weight matrix with singular values
// sigma_1..sigma_n, q_i = sigma_i^2 / sum_j sigma_j^2 and H = -(1 / log n) sum q_i log q_i.
//
// fp64 throughout. sigma_i^2 are the eigenvalues of the Gram matrix S = X X^T
// (X = W, or W^T for tall W, so S is min(A,B)^2):
//   k_sp_gram     S from fp32 W on the fp64 matrix cores (v_mfma_f64_16x16x4_f64);
//                 fp32 products are exact in fp64, so S carries fp64 accumulation error
//                 only. Upper block tiles, each stored twice, so S is exactly symmetric.
//   k_sp_house    column step j of the Householder tridiagonalisation: finishes the
//                 previous step's w, forms column j of the current matrix, the diagonal
//                 and sub-diagonal entries d_j, e_j, and the reflector (v_j, tau_j).
//   k_sp_pass     one sweep over the upper triangle of the trailing block, in 64 x 64
//                 tiles: applies the previous step's rank-2 update
//                 A <- A - v w^T - w v^T and, from the updated values, each tile's row
//                 sums of A v_j and (A symmetric) its column sums, into partial arrays.
//                 The upper triangle is read and written once per step: HBM-bound.
//   k_sp_reduce   p_j = tau_j A v_j from the tile partials, in a fixed order.
//   k_sp_bisect   eigenvalue k of the tridiagonal matrix by bisection on Sturm counts,
//                 one thread per eigenvalue, from the Gershgorin interval.
//   k_sp_entropy  normalisation, entropy, and the optional sigma^2 output.
// The rank-2 update is evaluated without contraction in a form that is symmetric in
// its two indices. Only the upper triangle of the trailing block is kept current, so
// row j (contiguous) is read where the method needs column j.
#include <float.h>

#include "launch.hpp"

namespace muon {

typedef double doublex4 __attribute__((ext_vector_type(4)));
typedef double doublex2 __attribute__((ext_vector_type(2)));

constexpr int kSpBK = 16;                // K slice per LDS stage
constexpr int kSpLdsLd = kSpTile + 16;   // LDS row stride (doubles): 4 k-rows of a
                                         // fragment read land in two bank halves

// s - (vr wc + wr vc), rounded step by step: swapping (r, c) swaps the operands of
// each product and of the sum, so element (c, r) gets the identical value.
__device__ __forceinline__ double rank2_sub(double s, double vr, double wc, double wr, double vc) {
#pragma clang fp contract(off)
    const double x = vr * wc;
    const double y = wr * vc;
    return s - (x + y);
}

// Fixed-order sum over a block of `kWaves` waves; every thread gets the result.
template <int kWaves>
__device__ __forceinline__ double block_sum_d(double v, double* red) {
    v = wave_sum_d(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) s += red[i];
    __syncthreads();
    return s;
}

// ------------------------------------------------------------------ Gram ----
// One 128 x 128 tile of S per block (upper tiles only), 4 waves of 64 x 64, each a
// 4 x 4 grid of 16 x 16 MFMA blocks. X tiles are staged k-major in LDS as fp64, so a
// fragment read is 16 consecutive doubles per k row. Operand layout of the 16x16x4
// f64 MFMA: A[i][k] in lane i + 16 k, B[k][j] in lane j + 16 k; result element r of
// lane l is D[l / 16 + 4 r][l % 16] (checked on the device with an in-bounds probe).
__global__ __launch_bounds__(256) void k_sp_gram(SpArgs args) {
    __shared__ double xs[2][kSpBK][kSpLdsLd];
    __shared__ double ys[2][kSpBK][kSpLdsLd];
    const int b = blockIdx.x;
    int mi = 0;
    while (mi + 1 < args.n && args.d[mi + 1].tile_begin <= b) ++mi;
    const SpDesc& d = args.d[mi];
    int local = b - d.tile_begin, ti = 0, row_len = d.tm;
    while (local >= row_len) {
        local -= row_len;
        ++ti;
        --row_len;
    }
    const int tj = ti + local;
    const int i0 = ti * kSpTile, j0 = tj * kSpTile;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = d.m, n = d.n;
    const int64_t ldw = d.cols;
    const float* w = d.w;
    const bool tall = d.tall != 0;

    // Thread t loads 8 elements of a 128 x 16 slice of X: flat X = W rows are
    // k-contiguous (row t / 2, k 8 (t % 2) ..), tall X = W^T rows are columns of W,
    // contiguous along i (k t / 16, i 8 (t % 16) ..). Out of range reads are zeros.
    auto load = [&](float* r, int base, int k0) {
        if (!tall) {
            const int i = base + (tid >> 1), k = k0 + (tid & 1) * 8;
            const float* src = w + (int64_t)i * ldw + k;
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = (i < m && k + e < n) ? src[e] : 0.f;
        } else {
            const int k = k0 + (tid >> 4), i = base + (tid & 15) * 8;
            const float* src = w + (int64_t)k * ldw + i;
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = (k < n && i + e < m) ? src[e] : 0.f;
        }
    };
    auto store = [&](double (*dst)[kSpLdsLd], const float* r) {
        if (!tall) {
            const int i = tid >> 1, k = (tid & 1) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[k + e][i] = (double)r[e];
        } else {
            const int k = tid >> 4, i = (tid & 15) * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[k][i + e] = (double)r[e];
        }
    };

    const int wr = wave >> 1, wc = wave & 1;
    doublex4 acc[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = doublex4{0.0, 0.0, 0.0, 0.0};

    float rx[8], ry[8];
    const int nk = (n + kSpBK - 1) / kSpBK;
    load(rx, i0, 0);
    load(ry, j0, 0);
    store(xs[0], rx);
    store(ys[0], ry);
    __syncthreads();
    for (int s = 0; s < nk; ++s) {
        const int cur = s & 1;
        if (s + 1 < nk) {
            load(rx, i0, (s + 1) * kSpBK);
            load(ry, j0, (s + 1) * kSpBK);
        }
#pragma unroll
        for (int kk = 0; kk < kSpBK / 4; ++kk) {
            const int kr = kk * 4 + (lane >> 4);
            double a[4], bv[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) a[p] = xs[cur][kr][wr * 64 + p * 16 + (lane & 15)];
#pragma unroll
            for (int q = 0; q < 4; ++q) bv[q] = ys[cur][kr][wc * 64 + q * 16 + (lane & 15)];
#pragma unroll
            for (int p = 0; p < 4; ++p)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[p][q] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[p], bv[q], acc[p][q], 0, 0, 0);
        }
        if (s + 1 < nk) {
            store(xs[cur ^ 1], rx);
            store(ys[cur ^ 1], ry);
        }
        __syncthreads();
    }

    double* S = d.s;
    const int64_t ld = d.ld;
    const bool diag = ti == tj;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t gi = i0 + wr * 64 + p * 16 + (lane >> 4) + 4 * r;
                const int64_t gj = j0 + wc * 64 + q * 16 + (lane & 15);
                const double v = acc[p][q][r];
                if (!diag) {
                    S[gi * ld + gj] = v;
                    S[gj * ld + gi] = v;
                } else if (gi <= gj) {  // diagonal tile: the upper half, mirrored
                    S[gi * ld + gj] = v;
                    S[gj * ld + gi] = v;
                }
            }
}

// ------------------------------------------------------------ Householder ----
// One 1024-thread block per matrix at column step j. Thread t owns the entries
// i = j + t + 1024 u. With v = v_{j-1}, p = p_{j-1}, tau = tau_{j-1}:
//   w_i   = p_i - (tau / 2) (p . v) v_i                     (stored for the pass)
//   col_i = S[j][i] - (v_i w_j + w_i v_j)                   (column j of the current A)
//   d_j = col_j; from x = col_{j+1..}: alpha = x_0, sigma2 = |x_{1..}|^2,
//   beta = -sign(alpha) sqrt(alpha^2 + sigma2), v_j = (1, x_{1..} / (alpha - beta)),
//   tau_j = (beta - alpha) / beta, e_j = beta  (tau_j = 0, e_j = alpha if sigma2 = 0).
// x_{1..} is parked in v_j's own entries between the two passes (each thread rereads
// only what it wrote).
__global__ __launch_bounds__(1024) void k_sp_house(SpArgs args) {
    __shared__ double red[16];
    __shared__ double alpha_s;
    const SpDesc& d = args.d[blockIdx.x];
    const int j = args.j, m = d.m, tid = threadIdx.x;
    if (j >= m) return;
    const double* vp = d.v[(j + 1) & 1];
    double* vc = d.v[j & 1];
    const double* srow = d.s + (int64_t)j * d.ld;
    const bool upd = j > 0;

    double kcoef = 0.0;
    if (upd) {
        double dot = 0.0;
        for (int i = j + tid; i < m; i += 1024) dot += d.p[i] * vp[i];
        kcoef = 0.5 * d.tau[(j + 1) & 1] * block_sum_d<16>(dot, red);
    }
    const double vj = upd ? vp[j] : 0.0;
    const double wj = upd ? d.p[j] - kcoef * vj : 0.0;
    double sig2 = 0.0;
    for (int i = j + tid; i < m; i += 1024) {
        double col = srow[i];
        if (upd) {
            const double wi = d.p[i] - kcoef * vp[i];
            d.wv[i] = wi;
            col = rank2_sub(col, vj, wi, wj, vp[i]);
        }
        if (i == j) d.d[j] = col;
        else if (i == j + 1) alpha_s = col;
        else {
            sig2 += col * col;
            vc[i] = col;
        }
    }
    if (j == m - 1) return;  // last diagonal entry: no reflector (uniform per block)
    sig2 = block_sum_d<16>(sig2, red);  // its barriers also publish alpha_s
    const double alpha = alpha_s;
    double tau = 0.0, beta = alpha, inv = 0.0;
    if (sig2 > 0.0) {
        const double mu = sqrt(alpha * alpha + sig2);
        beta = alpha >= 0.0 ? -mu : mu;
        tau = (beta - alpha) / beta;
        inv = 1.0 / (alpha - beta);
    }
    if (tid == 0) {
        d.tau[j & 1] = tau;
        d.e[j] = beta;
        vc[j + 1] = 1.0;
    }
    for (int i = j + tid; i < m; i += 1024)  // the same ownership as the first pass
        if (i >= j + 2) vc[i] = sig2 > 0.0 ? vc[i] * inv : 0.0;
}

// -------------------------------------------------------- trailing sweep ----
// Tile (I, J), I <= J, of the absolute 64 x 64 tiling over rows/columns [j+1, m) of
// matrix blockIdx.y; element (r, c) takes part iff j < r <= c < m. Thread t holds the
// column pair c = 64 J + 2 (t % 32) + {0, 1} on rows 64 I + t / 32 + 8 k, k < 8.
//   A[r][c] <- A[r][c] - (v_r w_c + w_r v_c)   (previous step's update, j > 0; stored)
//   rowpart[I][J][r % 64] = sum_c A[r][c] x_c        (x = v_j; all c of the tile)
//   colpart[I][J][c % 64] = sum_{r < c} A[r][c] x_r  (the mirrored lower element)
// Every tile of the active range writes all 64 entries of both partials (zeros where
// masked), so the reduce kernel reads no stale partial.
__global__ __launch_bounds__(256) void k_sp_pass(SpArgs args) {
    __shared__ double red[8][kSpPassTile];
    const SpDesc& d = args.d[blockIdx.y];
    const int j = args.j, m = d.m;
    if (j > m - 2) return;
    const int t0 = (j + 1) / kSpPassTile, tm = (m + kSpPassTile - 1) / kSpPassTile, nt = tm - t0;
    int local = blockIdx.x;
    if (local >= nt * (nt + 1) / 2) return;  // uniform per block
    int I = t0, len = nt;
    while (local >= len) {
        local -= len;
        ++I;
        --len;
    }
    const int J = I + local;
    const int tid = threadIdx.x, cp = tid & 31, rg = tid >> 5;
    const bool upd = j > 0;
    const double* vp = d.v[(j + 1) & 1];
    const double* x = d.v[j & 1];
    const double* wv = d.wv;
    const int64_t ld = d.ld;
    const int c0 = j + 1;
    const int c = J * kSpPassTile + 2 * cp;  // even, c + 1 < m_p
    const bool cok0 = c >= c0 && c < m, cok1 = c + 1 >= c0 && c + 1 < m;
    const doublex2 xc = *reinterpret_cast<const doublex2*>(x + c);
    doublex2 vcol = {0.0, 0.0}, wcol = {0.0, 0.0};
    if (upd) {
        vcol = *reinterpret_cast<const doublex2*>(vp + c);
        wcol = *reinterpret_cast<const doublex2*>(wv + c);
    }
    double col0 = 0.0, col1 = 0.0, rowp[8];
    const int rbase = I * kSpPassTile + rg;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = rbase + 8 * k;
        rowp[k] = 0.0;
        if (r < c0 || r >= m) continue;
        const bool e0 = cok0 && c >= r, e1 = cok1 && c + 1 >= r;
        if (!(e0 || e1)) continue;
        double* row = d.s + (int64_t)r * ld + c;
        doublex2 a = *reinterpret_cast<const doublex2*>(row);
        if (upd) {
            const double vr = vp[r], wr = wv[r];
            a.x = rank2_sub(a.x, vr, wcol.x, wr, vcol.x);
            a.y = rank2_sub(a.y, vr, wcol.y, wr, vcol.y);
            if (e0 && e1) *reinterpret_cast<doublex2*>(row) = a;
            else if (e0) row[0] = a.x;
            else row[1] = a.y;
        }
        const double xr = x[r];
        if (e0) {
            rowp[k] += a.x * xc.x;
            if (c > r) col0 += a.x * xr;
        }
        if (e1) {
            rowp[k] += a.y * xc.y;
            if (c + 1 > r) col1 += a.y * xr;
        }
    }
    const int64_t pbase = ((int64_t)I * d.tp + J) * kSpPassTile;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        double v = rowp[k];
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);  // the 32 lanes of one row
        if (cp == 0) d.rowpart[pbase + rg + 8 * k] = v;
    }
    red[rg][2 * cp] = col0;
    red[rg][2 * cp + 1] = col1;
    __syncthreads();
    if (tid < kSpPassTile) {
        double v = 0.0;
#pragma unroll
        for (int g = 0; g < 8; ++g) v += red[g][tid];
        d.colpart[pbase + tid] = v;
    }
}

// p_r = tau_j (sum_{J >= I} rowpart[I][J][r % 64] + sum_{t0 <= I' <= I} colpart[I'][I][r % 64])
// for rows r in [j+1, m), I = r / 64: row sums of the tiles right of the diagonal and
// column sums of the tiles above it, J and I' ascending.
__global__ __launch_bounds__(256) void k_sp_reduce(SpArgs args) {
    const SpDesc& d = args.d[blockIdx.y];
    const int j = args.j, m = d.m;
    const int r = j + 1 + blockIdx.x * 256 + threadIdx.x;
    if (j > m - 2 || r >= m) return;
    const int t0 = (j + 1) / kSpPassTile, tm = (m + kSpPassTile - 1) / kSpPassTile;
    const int I = r / kSpPassTile, lr = r % kSpPassTile;
    // four independent chains (J and I' ascending within each), combined at the end
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    const double* rp = d.rowpart + (int64_t)I * d.tp * kSpPassTile + lr;  // + J * 64
    int J = I;
    for (; J + 4 <= tm; J += 4) {
        s0 += rp[(int64_t)J * kSpPassTile];
        s1 += rp[(int64_t)(J + 1) * kSpPassTile];
        s2 += rp[(int64_t)(J + 2) * kSpPassTile];
        s3 += rp[(int64_t)(J + 3) * kSpPassTile];
    }
    for (; J < tm; ++J) s0 += rp[(int64_t)J * kSpPassTile];
    const double* cq = d.colpart + (int64_t)I * kSpPassTile + lr;  // + I' * tp * 64
    const int64_t cs = (int64_t)d.tp * kSpPassTile;
    int I2 = t0;
    for (; I2 + 4 <= I + 1; I2 += 4) {
        s0 += cq[I2 * cs];
        s1 += cq[(I2 + 1) * cs];
        s2 += cq[(I2 + 2) * cs];
        s3 += cq[(I2 + 3) * cs];
    }
    for (; I2 <= I; ++I2) s0 += cq[I2 * cs];
    d.p[r] = d.tau[j & 1] * ((s0 + s1) + (s2 + s3));
}

// ------------------------------------------------------------- bisection ----
// Number of eigenvalues of the tridiagonal (d, e) below x: negative pivots of the
// LDL^T factorisation of T - x I (Sturm sequence), tiny pivots replaced by -pivmin.
// e^2 / q is formed as e^2 * (1 / q) with the hardware reciprocal refined by two
// Newton steps r <- r + r (1 - q r), which reaches full double accuracy and is a
// quarter faster than the IEEE divide sequence on this dependency chain; |q| >= pivmin
// keeps q normal, and the count only needs q to a few ulps.
__device__ __forceinline__ int sturm_count(const double* dd, const double* ee, int m, double x,
                                           double pivmin) {
    double q = dd[0] - x;
    if (fabs(q) < pivmin) q = -pivmin;
    int c = q < 0.0;
    for (int i = 1; i < m; ++i) {
        const double e = ee[i - 1];
        double rq = __builtin_amdgcn_rcp(q);
        rq = fma(fma(-q, rq, 1.0), rq, rq);
        rq = fma(fma(-q, rq, 1.0), rq, rq);
        q = (dd[i] - x) - (e * e) * rq;
        if (fabs(q) < pivmin) q = -pivmin;
        c += q < 0.0;
    }
    return c;
}

// Eigenvalue k (ascending) of matrix blockIdx.y for k = blockIdx.x * 256 + thread.
// Invariant count(lo) <= k < count(hi), from the widened Gershgorin interval; halving
// stops when no double lies strictly inside or after kSpBisectIters steps (the width is
// then 2^-80 of the interval). A NaN anywhere in (d, e) makes every eigenvalue NaN.
__global__ __launch_bounds__(256) void k_sp_bisect(SpArgs args) {
    __shared__ double red[4][4];
    const SpDesc& d = args.d[blockIdx.y];
    const int m = d.m, tid = threadIdx.x;
    if ((int)blockIdx.x * 256 >= m) return;  // uniform per block
    double lo = DBL_MAX, hi = -DBL_MAX, e2max = 0.0, bad = 0.0;
    for (int i = tid; i < m; i += 256) {
        const double el = i > 0 ? fabs(d.e[i - 1]) : 0.0;
        const double er = i < m - 1 ? fabs(d.e[i]) : 0.0;
        const double di = d.d[i];
        lo = fmin(lo, di - (el + er));
        hi = fmax(hi, di + (el + er));
        e2max = fmax(e2max, er * er);
        if (di != di || er != er) bad = 1.0;  // fmin / fmax drop NaN: flag it
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = fmin(lo, __shfl_xor(lo, o, 64));
        hi = fmax(hi, __shfl_xor(hi, o, 64));
        e2max = fmax(e2max, __shfl_xor(e2max, o, 64));
        bad = fmax(bad, __shfl_xor(bad, o, 64));
    }
    const int wave = tid >> 6;
    if ((tid & 63) == 0) {
        red[0][wave] = lo;
        red[1][wave] = hi;
        red[2][wave] = e2max;
        red[3][wave] = bad;
    }
    __syncthreads();
    lo = fmin(fmin(red[0][0], red[0][1]), fmin(red[0][2], red[0][3]));
    hi = fmax(fmax(red[1][0], red[1][1]), fmax(red[1][2], red[1][3]));
    e2max = fmax(fmax(red[2][0], red[2][1]), fmax(red[2][2], red[2][3]));
    bad = fmax(fmax(red[3][0], red[3][1]), fmax(red[3][2], red[3][3]));
    const int k = blockIdx.x * 256 + tid;
    if (k >= m) return;
    if (bad != 0.0) {
        d.lam[k] = __builtin_nan("");
        return;
    }
    const double pivmin = DBL_MIN * fmax(1.0, e2max);
    const double widen = 4.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)) + 2.0 * pivmin;
    double a = lo - widen, b = hi + widen;
    for (int it = 0; it < kSpBisectIters; ++it) {
        const double mid = 0.5 * (a + b);
        if (!(mid > a && mid < b)) break;
        if (sturm_count(d.d, d.e, m, mid, pivmin) > k) b = mid;
        else a = mid;
    }
    d.lam[k] = 0.5 * (a + b);
}

// --------------------------------------------------------------- entropy ----
// One block per matrix: total = sum max(lambda, 0), q = lambda / total,
// H = -(sum q log q) / log m, with H = 0 for m = 1 and NaN when total is 0.
// Negative eigenvalues (rounding of a semi-definite S) count as 0; NaN propagates.
__device__ __forceinline__ double clamp0(double x) { return x < 0.0 ? 0.0 : x; }

__global__ __launch_bounds__(256) void k_sp_entropy(SpArgs args) {
    __shared__ double red[4];
    const SpDesc& d = args.d[blockIdx.x];
    const int m = d.m, tid = threadIdx.x;
    double t = 0.0;
    for (int k = tid; k < m; k += 256) t += clamp0(d.lam[k]);
    const double total = block_sum_d<4>(t, red);
    double h = 0.0;
    for (int k = tid; k < m; k += 256) {
        const double q = clamp0(d.lam[k]) / total;
        if (!(q <= 0.0)) h -= q * log(q);
    }
    h = block_sum_d<4>(h, red);
    if (tid == 0) {
        double hv;
        if (total == 0.0) hv = __builtin_nan("");
        else if (m == 1) hv = total == total ? 0.0 : total;
        else hv = h / log((double)m);
        *d.entropy = hv;
    }
    if (args.sigma_sq) {
        double* out = args.sigma_sq + d.sigma_off;
        for (int k = tid; k < m; k += 256) out[m - 1 - k] = clamp0(d.lam[k]);
    }
}

hipError_t launch_sp_gram(const SpArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_sp_gram, dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sp_house(const SpArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_sp_house, dim3(a.n), dim3(1024), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sp_pass(const SpArgs& a, int max_tiles, hipStream_t s) {
    hipLaunchKernelGGL(k_sp_pass, dim3(max_tiles, a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sp_reduce(const SpArgs& a, int max_trailing, hipStream_t s) {
    hipLaunchKernelGGL(k_sp_reduce, dim3((max_trailing + 255) / 256, a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sp_bisect(const SpArgs& a, int max_m, hipStream_t s) {
    hipLaunchKernelGGL(k_sp_bisect, dim3((max_m + 255) / 256, a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sp_entropy(const SpArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_sp_entropy, dim3(a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace muon
