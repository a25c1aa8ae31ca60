// HBM-bound kernels of the Muon step: momentum + Frobenius partials + bf16 working
// copies, the Frobenius finalise, and the RowNorm step (rows for flat and square
// matrices in one pass, columns for tall matrices in three short kernels).
//
// Method sources: "Muon is Scalable for LLM Training" Sec. 2.1 Eq. 1 (momentum) and
// the Newton-Schulz paragraph (X0 = M / ||M||_F); "Scaling Muon for Diffusion
// Transformers", Periodic Row-wise and distributed-implementation paragraphs
// (RowNorm of the current momentum: rows of flat matrices, per-column norms of tall
// ones). Every reduction runs in a fixed order, so results are bitwise repeatable.
#include "launch.hpp"

namespace muon {

template <typename Desc>
__device__ __forceinline__ int find_group(const Desc* d, int n, int t) {
    int g = 0;
    while (g + 1 < n && t >= d[g + 1].tile_begin) ++g;
    return g;
}

// ------------------------------------------------------------------ cast ----
// A matrix with no transposed copy (a tall one whose Gram reads X_c only) takes tiles of
// 16 rows x 256 columns, one wave per row: 1 KiB contiguous per row and array. On MI355X
// that pattern streams at 6.06 TB/s against 5.43 TB/s for the 64 x 64 tiles (256 bytes
// per row) that the transpose needs (a [30720, 5120] matrix, 14 bytes per element).
static_assert(kPad % 256 == 0, "a wide cast tile row spans 256 padded columns");
__device__ __forceinline__ void cast_wide(const CastArgs& args, const CastDesc& d, int local, float* red) {
    const int tiles_w = d.cols_p >> 8;
    const int tr = local / tiles_w, tc = local - tr * tiles_w;
    const int tid = threadIdx.x, lane = tid & 63, rq = tid >> 6;
    const int c0 = tc * 256 + lane * 4;
    const bool vec = (d.cols & 3) == 0;
    const bool mom = args.use_momentum != 0;
    const float mu = args.mu;
    float vv[4][4];
    if (vec) {
        floatx4 mm[4], gg[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = tr * 16 + rq + 4 * q;
            const bool ok = r < d.rows && c0 + 3 < d.cols;
            const int64_t o = (int64_t)r * d.cols + c0;
            mm[q] = ok ? ld_stream(d.m_in + o) : floatx4{0.f, 0.f, 0.f, 0.f};
            gg[q] = (ok && mom) ? ld_stream(d.g + o) : floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = tr * 16 + rq + 4 * q;
            const bool ok = r < d.rows && c0 + 3 < d.cols;
            floatx4 m = mm[q];
            if (mom) {
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = fmaf(mu, m[e], gg[q][e]);
            }
            if (ok && d.m_out) st_stream(d.m_out + (int64_t)r * d.cols + c0, m);
#pragma unroll
            for (int e = 0; e < 4; ++e) vv[q][e] = m[e];
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = tr * 16 + rq + 4 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c0 + e;
                float x = 0.f;
                if (r < d.rows && c < d.cols) {
                    const int64_t o = (int64_t)r * d.cols + c;
                    x = d.m_in[o];
                    if (mom) x = fmaf(mu, x, d.g[o]);
                    if (d.m_out) d.m_out[o] = x;
                }
                vv[q][e] = x;
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = tr * 16 + rq + 4 * q;
        unsigned short h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ss = fmaf(vv[q][e], vv[q][e], ss);
            h[e] = f2bf(vv[q][e]);
        }
        u32x2 packed;
        packed.x = pack2(h[0], h[1]);
        packed.y = pack2(h[2], h[3]);
        const int64_t o = d.direct_blk ? kb_off(r, c0, d.cols_p) : (int64_t)r * d.cols_p + c0;
        *reinterpret_cast<u32x2*>(d.direct + o) = packed;
    }
    const float s = block_sum_256(ss, red);
    if (tid == 0) d.partial[local] = s;
}

__global__ __launch_bounds__(256) void k_cast(CastArgs args) {
    __shared__ unsigned short tile[64][64 + 2];
    __shared__ float red[4];
    const int t = blockIdx.x;
    const int gi = find_group(args.d, args.n, t);
    const CastDesc& d = args.d[gi];
    const int local = t - d.tile_begin;
    if (d.wide) {
        cast_wide(args, d, local, red);
        return;
    }
    const int tr = local / d.tiles_c, tc = local - tr * d.tiles_c;
    const int tid = threadIdx.x;
    const int c4 = tid & 15, rq = tid >> 4;
    const int c0 = tc * 64 + c4 * 4;
    const bool vec = (d.cols & 3) == 0;
    const bool mom = args.use_momentum != 0;
    const float mu = args.mu;
    // All loads of the tile are issued before the first store: M' is stored through
    // one pointer and M / G read through others, so a store could otherwise keep the
    // compiler from moving the following loads ahead of it.
    float vv[4][4];
    if (vec) {
        floatx4 mm[4], gg[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = tr * 64 + rq + 16 * q;
            const bool ok = r < d.rows && c0 + 3 < d.cols;
            const int64_t o = (int64_t)r * d.cols + c0;
            mm[q] = ok ? ld_stream(d.m_in + o) : floatx4{0.f, 0.f, 0.f, 0.f};
            gg[q] = (ok && mom) ? ld_stream(d.g + o) : floatx4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = tr * 64 + rq + 16 * q;
            const bool ok = r < d.rows && c0 + 3 < d.cols;
            floatx4 m = mm[q];
            if (mom) {
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = fmaf(mu, m[e], gg[q][e]);
            }
            if (ok && d.m_out) st_stream(d.m_out + (int64_t)r * d.cols + c0, m);
#pragma unroll
            for (int e = 0; e < 4; ++e) vv[q][e] = m[e];
        }
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = tr * 64 + rq + 16 * q;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c0 + e;
                float x = 0.f;
                if (r < d.rows && c < d.cols) {
                    const int64_t o = (int64_t)r * d.cols + c;
                    x = d.m_in[o];
                    if (mom) x = fmaf(mu, x, d.g[o]);
                    if (d.m_out) d.m_out[o] = x;
                }
                vv[q][e] = x;
            }
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rl = rq + 16 * q;
        const int r = tr * 64 + rl;
        unsigned short h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ss = fmaf(vv[q][e], vv[q][e], ss);
            h[e] = f2bf(vv[q][e]);
            tile[rl][c4 * 4 + e] = h[e];
        }
        u32x2 packed;
        packed.x = pack2(h[0], h[1]);
        packed.y = pack2(h[2], h[3]);
        if (d.direct) {
            const int64_t o = d.direct_blk ? kb_off(r, c0, d.cols_p) : (int64_t)r * d.cols_p + c0;
            *reinterpret_cast<u32x2*>(d.direct + o) = packed;
        }
    }
    __syncthreads();
    if (d.transp) {
        // transposed copy: output row = input column oc, 16 consecutive input rows
        const int oc = tid >> 2, ob = (tid & 3) * 16;
        unsigned w8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w8[e] = pack2(tile[ob + 2 * e][oc], tile[ob + 2 * e + 1][oc]);
        unsigned short* dst = d.transp + (d.transp_blk ? kb_off(tc * 64 + oc, tr * 64 + ob, d.rows_p)
                                                       : (int64_t)(tc * 64 + oc) * d.rows_p + tr * 64 + ob);
        u32x4 lo, hi;
        lo.x = w8[0]; lo.y = w8[1]; lo.z = w8[2]; lo.w = w8[3];
        hi.x = w8[4]; hi.y = w8[5]; hi.z = w8[6]; hi.w = w8[7];
        reinterpret_cast<u32x4*>(dst)[0] = lo;
        reinterpret_cast<u32x4*>(dst)[1] = hi;
    }
    const float s = block_sum_256(ss, red);
    if (tid == 0) d.partial[local] = s;
}

hipError_t launch_cast(const CastArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_cast, dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ frob ----
__global__ __launch_bounds__(256) void k_frob(FrobArgs args) {
    __shared__ double red[4];
    const int g = blockIdx.x;
    const float* p = args.partial[g];
    const int n = args.count[g];
    double acc = 0.0;
    for (int i = threadIdx.x; i < n; i += 256) acc += (double)p[i];
    acc = wave_sum_d(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double tot = (red[0] + red[1]) + (red[2] + red[3]);
        const float nrm = (float)sqrt(tot);
        *args.scale[g] = 1.0f / max_keep_nan(nrm, args.eps);
    }
}

hipError_t launch_frob(const FrobArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_frob, dim3(a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

// --------------------------------------------------------- rownorm (rows) ----
// One 256-thread block per row; the row's M' stays in registers between the norm
// reduction and the weight update, so every element moves exactly once:
// read M, G, W and write M, W (20 bytes per element).
template <int VMAX, bool VEC>
__global__ __launch_bounds__(256) void k_rownorm_rows(RowArgs args) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].row_begin) ++gi;
    const RowDesc& d = args.d[gi];
    const int row = t - d.row_begin;
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)row * d.cols;
    const float mu = args.mu;
    float ss = 0.f;
    if constexpr (VEC) {
        // Loads are issued in batches of kB float4 ahead of the batch's stores (M' is
        // written through a pointer that the compiler cannot prove distinct from G's).
        constexpr int kB = 4;
        floatx4 mv[VMAX];
        const float* gp = d.g + base;
        float* mp = d.m + base;
        float* wp = d.w + base;
        const int nv = d.cols >> 2;
#pragma unroll
        for (int k0 = 0; k0 < VMAX; k0 += kB) {
            floatx4 gv[kB];
#pragma unroll
            for (int k = k0; k < k0 + kB && k < VMAX; ++k) {
                const int idx = k * 256 + tid;
                if (idx < nv) {
                    mv[k] = ld_stream(mp + 4 * idx);
                    gv[k - k0] = ld_stream(gp + 4 * idx);
                }
            }
#pragma unroll
            for (int k = k0; k < k0 + kB && k < VMAX; ++k) {
                const int idx = k * 256 + tid;
                if (idx < nv) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        mv[k][e] = fmaf(mu, mv[k][e], gv[k - k0][e]);
                        ss = fmaf(mv[k][e], mv[k][e], ss);
                    }
                    st_stream(mp + 4 * idx, mv[k]);
                }
            }
        }
        const float tot = block_sum_256(ss, red);
        const float den = max_keep_nan(sqrtf(tot), args.eps);
        const float c = d.coef / den;
        if (d.part && tid == 0) d.part[row] = tot / (den * den);
        const float decay = args.decay;
#pragma unroll
        for (int k0 = 0; k0 < VMAX; k0 += kB) {
            floatx4 wv[kB];
#pragma unroll
            for (int k = k0; k < k0 + kB && k < VMAX; ++k) {
                const int idx = k * 256 + tid;
                if (idx < nv) wv[k - k0] = ld_stream(wp + 4 * idx);
            }
#pragma unroll
            for (int k = k0; k < k0 + kB && k < VMAX; ++k) {
                const int idx = k * 256 + tid;
                if (idx < nv) {
                    floatx4 w = wv[k - k0];
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = fmaf(-c, mv[k][e], w[e] * decay);
                    st_stream(wp + 4 * idx, w);
                }
            }
        }
    } else {
        float mv[VMAX * 4];
#pragma unroll
        for (int k = 0; k < VMAX * 4; ++k) {
            const int idx = k * 256 + tid;
            if (idx < d.cols) {
                const float m = fmaf(mu, d.m[base + idx], d.g[base + idx]);
                d.m[base + idx] = m;
                mv[k] = m;
                ss = fmaf(m, m, ss);
            }
        }
        const float tot = block_sum_256(ss, red);
        const float den = max_keep_nan(sqrtf(tot), args.eps);
        const float c = d.coef / den;
        if (d.part && tid == 0) d.part[row] = tot / (den * den);
        const float decay = args.decay;
#pragma unroll
        for (int k = 0; k < VMAX * 4; ++k) {
            const int idx = k * 256 + tid;
            if (idx < d.cols) d.w[base + idx] = fmaf(-c, mv[k], d.w[base + idx] * decay);
        }
    }
}

// Wide rows (kRowWideCols < cols <= kRowMaxRegisterCols, cols a multiple of 4): one
// 1024-thread block per row, VMAX float4 of M' per thread. All of a thread's M and G
// loads go out in one batch, and its W loads before the row reduction, so the block
// waits on memory once per phase. On MI355X a [5120, 20480] matrix streams at 5.9 TB/s
// this way against 5.45 TB/s with 256-thread blocks that hold 20 float4 each. The row
// sum adds each thread's values in index order, then the 64 lanes, then the 16 waves in
// a fixed tree.
template <int VMAX>
__global__ __launch_bounds__(1024) void k_rownorm_rows_wide(RowArgs args) {
    __shared__ float red[16];
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].row_begin) ++gi;
    const RowDesc& d = args.d[gi];
    const int row = t - d.row_begin;
    const int tid = threadIdx.x;
    const int64_t base = (int64_t)row * d.cols;
    const float* __restrict__ gp = d.g + base;
    float* __restrict__ mp = d.m + base;
    float* __restrict__ wp = d.w + base;
    const int nv = d.cols >> 2;
    const float mu = args.mu;
    floatx4 mv[VMAX], gv[VMAX], wv[VMAX];
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
        const int idx = k * 1024 + tid;
        if (idx < nv) {
            mv[k] = ld_stream(mp + 4 * idx);
            gv[k] = ld_stream(gp + 4 * idx);
        }
    }
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
        const int idx = k * 1024 + tid;
        if (idx < nv) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                mv[k][e] = fmaf(mu, mv[k][e], gv[k][e]);
                ss = fmaf(mv[k][e], mv[k][e], ss);
            }
            st_stream(mp + 4 * idx, mv[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
        const int idx = k * 1024 + tid;
        if (idx < nv) wv[k] = ld_stream(wp + 4 * idx);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = red[2 * i] + red[2 * i + 1];
    const float tot = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
    const float den = max_keep_nan(sqrtf(tot), args.eps);
    const float c = d.coef / den;
    if (d.part && tid == 0) d.part[row] = tot / (den * den);
    const float decay = args.decay;
#pragma unroll
    for (int k = 0; k < VMAX; ++k) {
        const int idx = k * 1024 + tid;
        if (idx < nv) {
            floatx4 w = wv[k];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = fmaf(-c, mv[k][e], w[e] * decay);
            st_stream(wp + 4 * idx, w);
        }
    }
}

hipError_t launch_rownorm_rows_wide(const RowArgs& a, int max_cols, hipStream_t s) {
    const dim3 grid(a.total), block(1024);
    const int need = (max_cols + 4095) / 4096;  // float4 per thread
    if (need <= 4) hipLaunchKernelGGL(k_rownorm_rows_wide<4>, grid, block, 0, s, a);
    else if (need <= 5) hipLaunchKernelGGL(k_rownorm_rows_wide<5>, grid, block, 0, s, a);
    else if (need <= 6) hipLaunchKernelGGL(k_rownorm_rows_wide<6>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(k_rownorm_rows_wide<8>, grid, block, 0, s, a);
    return hipGetLastError();
}

// Rows longer than the register budget: M' is written, then re-read for the update.
__global__ __launch_bounds__(256) void k_rownorm_rows_long(RowArgs args) {
    __shared__ float red[4];
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].row_begin) ++gi;
    const RowDesc& d = args.d[gi];
    const int row = t - d.row_begin;
    const int64_t base = (int64_t)row * d.cols;
    float ss = 0.f;
    for (int idx = threadIdx.x; idx < d.cols; idx += 256) {
        const float m = fmaf(args.mu, d.m[base + idx], d.g[base + idx]);
        d.m[base + idx] = m;
        ss = fmaf(m, m, ss);
    }
    // each thread re-reads only the elements it wrote itself, so no fence is needed
    const float tot = block_sum_256(ss, red);
    const float den = max_keep_nan(sqrtf(tot), args.eps);
    const float c = d.coef / den;
    if (d.part && threadIdx.x == 0) d.part[row] = tot / (den * den);
    for (int idx = threadIdx.x; idx < d.cols; idx += 256)
        d.w[base + idx] = fmaf(-c, d.m[base + idx], d.w[base + idx] * args.decay);
}

// Rows of 1024 to 8192 floats stream faster with fewer of them in flight per compute
// unit: a [*, 5120] set moves 6.29 TB/s at three blocks per compute unit against 5.75
// TB/s at the register-limited seven (2048: 6.63 against 6.03; 8192: 5.96 against
// 5.75). Unused dynamic LDS sets that limit; rows up to 1024 floats keep every block.
constexpr size_t kRowLdsCap = 40 * 1024;

hipError_t launch_rownorm_rows(const RowArgs& a, int max_cols, bool vec, hipStream_t s) {
    const dim3 grid(a.total), block(256);
    if (max_cols > kRowMaxRegisterCols) {
        hipLaunchKernelGGL(k_rownorm_rows_long, grid, block, 0, s, a);
    } else if (vec) {
        const int need = (max_cols + 1023) / 1024;  // float4 per thread
        const size_t lds = need > 1 ? kRowLdsCap : 0;
        if (need <= 2) hipLaunchKernelGGL((k_rownorm_rows<2, true>), grid, block, lds, s, a);
        else if (need <= 4) hipLaunchKernelGGL((k_rownorm_rows<4, true>), grid, block, lds, s, a);
        else if (need <= 8) hipLaunchKernelGGL((k_rownorm_rows<8, true>), grid, block, lds, s, a);
        else hipLaunchKernelGGL(k_rownorm_rows_long, grid, block, 0, s, a);  // wider rows take the wide kernel
    } else {
        const int need = (max_cols + 1023) / 1024;
        if (need <= 2) hipLaunchKernelGGL((k_rownorm_rows<2, false>), grid, block, 0, s, a);
        else if (need <= 8) hipLaunchKernelGGL((k_rownorm_rows<8, false>), grid, block, 0, s, a);
        else hipLaunchKernelGGL(k_rownorm_rows_long, grid, block, 0, s, a);
    }
    return hipGetLastError();
}

// ------------------------------------------------------ colnorm (tall) ------
// Block tile: kColChunkRows rows x kColTileCols columns. Thread layout: 64 lanes
// cover 256 consecutive columns (one float4 each), the 4 waves interleave rows.
template <bool VEC>
__global__ __launch_bounds__(256) void k_colnorm_partial(ColArgs args) {
    __shared__ float red[4][kColTileCols];
    const int t = blockIdx.x;
    const int gi = find_group(args.d, args.n, t);
    const ColDesc& d = args.d[gi];
    const int local = t - d.tile_begin;
    const int chunk = local / d.tiles_c, tcol = local - chunk * d.tiles_c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = tcol * kColTileCols + lane * 4;
    const int r0 = chunk * kColChunkRows;
    const int r1 = min(r0 + kColChunkRows, d.rows);
    const float mu = args.mu;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if (VEC && c0 + 3 < d.cols) {
        // rows in batches of kB, loads ahead of stores (16: each wave's 16 rows of the
        // 64-row chunk in one batch)
        constexpr int kB = 16;
        for (int rb = r0 + wave; rb < r1; rb += 4 * kB) {
            floatx4 mv[kB], gv[kB];
#pragma unroll
            for (int q = 0; q < kB; ++q) {
                const int r = rb + 4 * q;
                if (r < r1) {
                    const int64_t o = (int64_t)r * d.cols + c0;
                    mv[q] = ld_stream(d.m + o);
                    gv[q] = ld_stream(d.g + o);
                }
            }
#pragma unroll
            for (int q = 0; q < kB; ++q) {
                const int r = rb + 4 * q;
                if (r < r1) {
                    floatx4 m = mv[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) m[e] = fmaf(mu, m[e], gv[q][e]);
                    st_stream(d.m + (int64_t)r * d.cols + c0, m);
                    s0 = fmaf(m[0], m[0], s0);
                    s1 = fmaf(m[1], m[1], s1);
                    s2 = fmaf(m[2], m[2], s2);
                    s3 = fmaf(m[3], m[3], s3);
                }
            }
        }
    } else {
        float sv[4] = {0.f, 0.f, 0.f, 0.f};
        for (int r = r0 + wave; r < r1; r += 4) {
            const int64_t o = (int64_t)r * d.cols;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c0 + e;
                if (c < d.cols) {
                    const float m = fmaf(mu, d.m[o + c], d.g[o + c]);
                    d.m[o + c] = m;
                    sv[e] = fmaf(m, m, sv[e]);
                }
            }
        }
        s0 = sv[0]; s1 = sv[1]; s2 = sv[2]; s3 = sv[3];
    }
    red[wave][lane * 4 + 0] = s0;
    red[wave][lane * 4 + 1] = s1;
    red[wave][lane * 4 + 2] = s2;
    red[wave][lane * 4 + 3] = s3;
    __syncthreads();
    const int c = tcol * kColTileCols + tid;
    if (c < d.cols)
        d.partial[(int64_t)chunk * d.cols + c] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

// One block per kColFinCols columns of a matrix: wave w adds the column's chunk partials
// of chunks [w q, (w + 1) q), q = ceil(chunks / 4), in chunk order (loads eight chunks
// ahead); the four wave sums are then added as (s0 + s1) + (s2 + s3). The order is
// fixed, so the norms are repeatable, and a single chunk's sum passes through exactly.
__global__ __launch_bounds__(256) void k_colnorm_finalize(ColArgs args) {
    static_assert(kColFinCols == 64, "one wave-wide column strip per block");
    __shared__ float red[4][kColFinCols];
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].fin_begin) ++gi;
    const ColDesc& d = args.d[gi];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = (t - d.fin_begin) * kColFinCols + lane;
    const int q = (d.chunks + 3) >> 2, k0 = wave * q, k1 = min(k0 + q, d.chunks);
    float s = 0.f;
    if (c < d.cols) {
        int k = k0;
        for (; k + 8 <= k1; k += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = d.partial[(int64_t)(k + j) * d.cols + c];
#pragma unroll
            for (int j = 0; j < 8; ++j) s += v[j];
        }
        for (; k < k1; ++k) s += d.partial[(int64_t)k * d.cols + c];
    }
    red[wave][lane] = s;
    __syncthreads();
    if (wave != 0 || c >= d.cols) return;
    s = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    if (args.sums_only) {  // a row block's share of a sharded matrix: the caller reduces
        d.inv[c] = s;
        return;
    }
    const float den = max_keep_nan(sqrtf(s), args.eps);
    d.inv[c] = 1.0f / den;
    if (d.part) d.part[c] = s / (den * den);
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_colnorm_apply(ColArgs args) {
    const int t = blockIdx.x;
    const int gi = find_group(args.d, args.n, t);
    const ColDesc& d = args.d[gi];
    const int local = t - d.tile_begin;
    const int chunk = local / d.tiles_c, tcol = local - chunk * d.tiles_c;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c0 = tcol * kColTileCols + lane * 4;
    const int r0 = chunk * kColChunkRows;
    const int r1 = min(r0 + kColChunkRows, d.rows);
    const float decay = args.decay;
    if (VEC && c0 + 3 < d.cols) {
        const floatx4 iv = *reinterpret_cast<const floatx4*>(d.inv + c0);
        floatx4 kc;
#pragma unroll
        for (int e = 0; e < 4; ++e) kc[e] = d.coef * iv[e];
        constexpr int kB = 16;
        for (int rb = r0 + wave; rb < r1; rb += 4 * kB) {
            floatx4 mv[kB], wv[kB];
#pragma unroll
            for (int q = 0; q < kB; ++q) {
                const int r = rb + 4 * q;
                if (r < r1) {
                    const int64_t o = (int64_t)r * d.cols + c0;
                    mv[q] = ld_stream(d.m + o);
                    wv[q] = ld_stream(d.w + o);
                }
            }
#pragma unroll
            for (int q = 0; q < kB; ++q) {
                const int r = rb + 4 * q;
                if (r < r1) {
                    floatx4 w = wv[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = fmaf(-kc[e], mv[q][e], w[e] * decay);
                    st_stream(d.w + (int64_t)r * d.cols + c0, w);
                }
            }
        }
    } else {
        float kc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kc[e] = (c0 + e < d.cols) ? d.coef * d.inv[c0 + e] : 0.f;
        for (int r = r0 + wave; r < r1; r += 4) {
            const int64_t o = (int64_t)r * d.cols;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c0 + e;
                if (c < d.cols) d.w[o + c] = fmaf(-kc[e], d.m[o + c], d.w[o + c] * decay);
            }
        }
    }
}

hipError_t launch_colnorm_partial(const ColArgs& a, bool vec, hipStream_t s) {
    if (vec) hipLaunchKernelGGL(k_colnorm_partial<true>, dim3(a.total), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_colnorm_partial<false>, dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_colnorm_finalize(const ColArgs& a, int fin_total, hipStream_t s) {
    hipLaunchKernelGGL(k_colnorm_finalize, dim3(fin_total), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_colnorm_apply(const ColArgs& a, bool vec, hipStream_t s) {
    if (vec) hipLaunchKernelGGL(k_colnorm_apply<true>, dim3(a.total), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_colnorm_apply<false>, dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ------------------------------------------------------- update RMS ----
// One block per matrix: RMS(U) from the partial sums of U^2 (fixed order, double),
// then the monitor value and, for the Eq. 6 rule ("Muon is Scalable for LLM
// Training", Sec. 3.1 Eq. 6), the per-matrix update coefficient lr * 0.2 / RMS(O).
__global__ __launch_bounds__(256) void k_rms_finalize(RmsArgs args) {
    __shared__ double red[4];
    const RmsDesc& d = args.d[blockIdx.x];
    double acc = 0.0;
    for (int i = threadIdx.x; i < d.count; i += 256) acc += (double)d.part[i];
    acc = wave_sum_d(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double tot = (red[0] + red[1]) + (red[2] + red[3]);
        const double r = sqrt(tot / d.elems);
        double mon;
        if (d.eq6) {
            const double den = r < (double)args.eps ? (double)args.eps : r;  // NaN stays NaN
            *d.coef_out = (float)((double)args.lr * (double)args.rms_scale / den);
            mon = (double)args.rms_scale * r / den;
        } else {
            mon = (double)d.dir_scale * r;
        }
        if (d.rms_out) *d.rms_out = (float)mon;
    }
}

hipError_t launch_rms_finalize(const RmsArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_rms_finalize, dim3(a.n), dim3(256), 0, s, a);
    return hipGetLastError();
}

// W <- decay W - coef O, the Eq. 6 update once RMS(O) is known. 16 elements per
// thread as four float4, loads of a block issued before its stores.
__global__ __launch_bounds__(256) void k_scaled_update(UpdArgs args) {
    const int t = blockIdx.x;
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].blk_begin) ++gi;
    const UpdDesc& d = args.d[gi];
    const float coef = *d.coef, decay = args.decay;
    const int64_t base = (int64_t)(t - d.blk_begin) * kUpdBlockElems;
    constexpr int kV = kUpdBlockElems / 256 / 4;
    if (base + kUpdBlockElems <= d.elems) {
        floatx4 ov[kV], wv[kV];
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int64_t i = base + (int64_t)(k * 256 + threadIdx.x) * 4;
            ov[k] = ld_stream(d.o + i);
            wv[k] = ld_stream(d.w + i);
        }
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int64_t i = base + (int64_t)(k * 256 + threadIdx.x) * 4;
            floatx4 w = wv[k];
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = fmaf(-coef, ov[k][e], w[e] * decay);
            st_stream(d.w + i, w);
        }
    } else {
        for (int64_t i = base + threadIdx.x; i < d.elems; i += 256) d.w[i] = fmaf(-coef, d.o[i], d.w[i] * decay);
    }
}

hipError_t launch_scaled_update(const UpdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_scaled_update, dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace muon
