// Newton-Schulz GEMM stage kernel template ("Muon is Scalable for LLM Training",
// Sec. 2.1 Eq. 2: X <- a X + b (X X^T) X + c (X X^T)^2 X).
//
// Each iteration is three products, all of the form C[i][j] = sum_k P[i][k] Q[j][k]
// with both operands K-contiguous in HBM:
//   Gram  A = X X^T   P = Q = X_r ([m_p, n_p])       K = n_p   symmetric output
//   Poly  B = bA+cAA  P = Q = A   ([m_p, m_p])       K = m_p   symmetric (A = A^T)
//   Apply X' = aX+BX  P = B, Q = X_c ([n_p, m_p])    K = m_p   X'_r and X'_c out
// Symmetric outputs compute only upper-triangular tiles and store each tile twice
// (mirrored). The first iteration folds s = 1 / ||M||_F into the Gram (s^2) and
// Apply (s) epilogues. The last Apply writes fp32 O in the input's orientation, or
// applies Eq. 4 to W directly.
//
// Block: 256 threads = 2 x 2 waves, each wave a (BM/2) x (BN/2) sub-tile built from
// v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulation). K step 64 bf16 = 128-byte
// LDS rows; the 16-byte chunk c of row r is stored at chunk position
// c ^ ((r >> 1) & 7). The LDS serves a 16-byte-per-lane read 16 lanes (256 bytes,
// all 64 banks) at a time; with this swizzle the 16 rows read by such a group land
// on 16 distinct 16-byte bank groups (measured: a plain (r & 7) swizzle left half
// of the LDS cycles in bank-conflict stalls).
//
// Tile order: consecutive blocks (which run together on one XCD after the remap)
// cover compact 2-D patches so that they share operand panels in L2: rectangular
// stages walk groups of 8 tile-rows column by column, symmetric stages walk 4 x 4
// super-tiles of the upper triangle.
// Operand tiles are double-buffered in LDS, one barrier per K step. Two ways to
// fill them:
//   kDirect = false: global -> VGPR -> LDS (ds_write_b128), loads for step k+1 in
//                    flight while step k computes;
//   kDirect = true:  global_load_lds_dwordx4 (gfx950): each lane's 16 bytes land at
//                    LDS base + 16 * lane, so lane l fetches the logical chunk that
//                    belongs at that swizzled position.
#pragma once

#include "launch.hpp"

namespace muon {

template <int BM_, int BN_, bool kDirect_, int BK_ = 64, int STAGES_ = 2>
struct GemmCfg {
    static constexpr int BM = BM_;
    static constexpr int BN = BN_;
    static constexpr bool kDirect = kDirect_;
    static constexpr int BK = BK_;
    static constexpr int STAGES = STAGES_;
    static constexpr int NT = 256;
    static constexpr int WM = BM / 2;
    static constexpr int WN = BN / 2;
    static constexpr int TM = WM / 32;
    static constexpr int TN = WN / 32;
    static constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row
    static constexpr int RB = BK * 2;             // bytes per LDS row
    static constexpr int RPI = 1024 / RB;         // rows per 1 KiB wave-wide load
    static constexpr int SWS = (RB == 128) ? 1 : 2;  // log2(rows per 256-byte bank window)
    static constexpr int LA = BM * CPR / NT;      // chunks per thread (register-staged path)
    static constexpr int LB = BN * CPR / NT;
    static constexpr int IA = BM / RPI / 4;       // 1 KiB loads per wave per stage (direct path)
    static constexpr int IB = BN / RPI / 4;
    static constexpr int kLdsBytes = STAGES * (BM + BN) * BK * 2;
    static_assert(BK == 32 || BK == 64, "K step");
    static_assert(kDirect || STAGES == 2, "the register-staged path is double-buffered");
};

// Element offset of logical 16-byte chunk `chunk` of LDS row `row`. The 16 rows that
// one 16-lane group reads sit in 16 / (256 / RB) bank windows; XOR-ing the chunk
// with (row >> SWS) spreads them over all 16 bank groups of 16 bytes.
template <class Cfg>
__device__ __forceinline__ int gemm_swz(int row, int chunk) {
    return row * Cfg::BK + ((chunk ^ ((row >> Cfg::SWS) & (Cfg::CPR - 1))) << 3);
}

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads(): that fence waits
// for every outstanding global load, which would drain the LDS prefetch queue each
// K step. The callers order their own memory: each wave waits (vmcnt) for its
// loads of the step about to be read, and every LDS read of the previous step has
// been consumed by an MFMA before the wave arrives here.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

constexpr int kRasterGroup = 8;  // rectangular: tile-rows per group
constexpr int kSuperTile = 4;    // symmetric: super-tile side

// local -> (ti, tj) for a tiles_m x tiles_n grid, groups of kRasterGroup tile-rows,
// each group walked column by column.
__device__ __forceinline__ void rect_tile(int local, int tiles_m, int tiles_n, int& ti, int& tj) {
    const int per = kRasterGroup * tiles_n;
    const int g = local / per;
    const int first = g * kRasterGroup;
    const int gs = min(tiles_m - first, kRasterGroup);
    const int r = local - g * per;
    ti = first + r % gs;
    tj = r / gs;
}

// local -> (ti <= tj) over the upper triangle of a T x T grid, in kSuperTile-sided
// super-tiles (row-major over the upper super-triangle, row-major inside).
__device__ __forceinline__ void tri_tile(int local, int T, int& ti, int& tj) {
    const int S = (T + kSuperTile - 1) / kSuperTile;
    int rem = local;
    for (int si = 0; si < S; ++si) {
        const int hi = min(kSuperTile, T - si * kSuperTile);
        for (int sj = si; sj < S; ++sj) {
            const int wj = min(kSuperTile, T - sj * kSuperTile);
            const int cnt = (si == sj) ? hi * (hi + 1) / 2 : hi * wj;
            if (rem < cnt) {
                if (si == sj) {
                    int a = 0;
                    while (rem >= hi - a) { rem -= hi - a; ++a; }
                    ti = si * kSuperTile + a;
                    tj = ti + rem;
                } else {
                    ti = si * kSuperTile + rem / wj;
                    tj = sj * kSuperTile + rem % wj;
                }
                return;
            }
            rem -= cnt;
        }
    }
    ti = tj = 0;  // not reached for local < T (T + 1) / 2
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

template <int MODE, class Cfg>
__device__ __forceinline__ void ns_gemm_tile(const NsArgs& args, unsigned short* sA, unsigned short* sB) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int STAGE_A = BM * BK, STAGE_B = BN * BK;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int t = xcd_remap(blockIdx.x, args.total);
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].tile_begin) ++gi;
    const NsDesc& d = args.d[gi];
    int local = t - d.tile_begin;

    constexpr bool kSym = (MODE == kModeGram || MODE == kModePoly);
    int ti, tj;
    if constexpr (kSym) tri_tile(local, d.tiles, ti, tj);
    else rect_tile(local, d.m_p / BM, d.tiles, ti, tj);

    const unsigned short* P;
    const unsigned short* Q;
    int64_t ld;
    int K;
    if constexpr (MODE == kModeGram) { P = d.xr; Q = d.xr; ld = d.n_p; K = d.n_p; }
    else if constexpr (MODE == kModePoly) { P = d.a; Q = d.a; ld = d.m_p; K = d.m_p; }
    else { P = d.b; Q = d.xc; ld = d.m_p; K = d.m_p; }
    const unsigned short* Pt = P + (int64_t)ti * BM * ld;
    const unsigned short* Qt = Q + (int64_t)tj * BN * ld;

    floatx16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int nk = K / BK;

    if constexpr (Cfg::kDirect) {
        // 1 KiB load j covers rows RPI*j .. RPI*j + RPI-1: lane l lands on row
        // RPI*j + l / CPR at physical chunk l % CPR, so it fetches the logical chunk that
        // the swizzle stores there (the XOR is its own inverse).
        constexpr int STAGES = Cfg::STAGES, RPI = Cfg::RPI, CPR = Cfg::CPR;
        constexpr int LOADS = Cfg::IA + Cfg::IB;  // wave-wide loads per K step
        constexpr int KK = BK / 16;               // MFMA sub-steps per K step
        constexpr int NMF = TM * TN;              // MFMAs per sub-step
        constexpr int NFR = TM + TN;              // fragment reads per sub-step
        constexpr int LPS = (LOADS + KK - 2) / (KK - 1);  // global loads per sub-step
        static_assert(KK >= 2 && KK % 2 == 0, "sub-step parity must restart at 0 every K step");
        static_assert(NFR <= NMF && 2 * LPS <= NMF, "issue slots");
        // the wave index is uniform: keep it scalar so the LDS destinations (M0) are too
        const int swave = __builtin_amdgcn_readfirstlane(wave);
        const int lrow = lane / CPR, lpc = lane % CPR;
        int64_t offa[Cfg::IA], offb[Cfg::IB];
#pragma unroll
        for (int q = 0; q < Cfg::IA; ++q) {
            const int row = (swave * Cfg::IA + q) * RPI + lrow;
            offa[q] = (int64_t)row * ld + ((lpc ^ ((row >> Cfg::SWS) & (CPR - 1))) << 3);
        }
#pragma unroll
        for (int q = 0; q < Cfg::IB; ++q) {
            const int row = (swave * Cfg::IB + q) * RPI + lrow;
            offb[q] = (int64_t)row * ld + ((lpc ^ ((row >> Cfg::SWS) & (CPR - 1))) << 3);
        }
        auto gload = [&](int buf, int k0, int idx) {  // idx < LOADS: one 1 KiB load
            if (idx < Cfg::IA)
                __builtin_amdgcn_global_load_lds((gbl_ptr_t)(Pt + offa[idx] + k0),
                                                 (lds_ptr_t)(sA + buf * STAGE_A + (swave * Cfg::IA + idx) * 512),
                                                 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds(
                    (gbl_ptr_t)(Qt + offb[idx - Cfg::IA] + k0),
                    (lds_ptr_t)(sB + buf * STAGE_B + (swave * Cfg::IB + idx - Cfg::IA) * 512), 16, 0, 0);
        };
        // Fragments are double-buffered in registers.
        bf16x8 fa[2][TM], fb[2][TN];
        auto frag = [&](int fbuf, int stage, int kk, int r) {  // r < NFR: one 16-byte read
            const int ch = kk * 2 + (lane >> 5);
            if (r < TM)
                fa[fbuf][r] = *reinterpret_cast<const bf16x8*>(
                    sA + stage * STAGE_A + gemm_swz<Cfg>(wm * WM + r * 32 + (lane & 31), ch));
            else
                fb[fbuf][r - TM] = *reinterpret_cast<const bf16x8*>(
                    sB + stage * STAGE_B + gemm_swz<Cfg>(wn * WN + (r - TM) * 32 + (lane & 31), ch));
        };
        // wait until this wave's loads of K step `st` are complete, given that steps
        // up to `last_issued` have been issued (loads complete in issue order)
        auto wait_step = [&](int st, int last_issued) {
            if (last_issued - st >= STAGES - 2) wait_vmcnt<LOADS * (STAGES - 2)>();
            else wait_vmcnt<0>();
        };
        // prologue: STAGES - 1 K steps in flight, then step 0's first fragments
#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            if (st < nk)
#pragma unroll
                for (int idx = 0; idx < LOADS; ++idx) gload(st, st * BK, idx);
        wait_step(0, min(STAGES - 2, nk - 1));
        barrier_no_fence();
#pragma unroll
        for (int r = 0; r < NFR; ++r) frag(0, 0, 0, r);
        // Main loop. Each MFMA occupies the matrix pipe for 8 passes; the wave issues at
        // most one LDS read and one global load between two MFMAs, so the other issue
        // work hides in the MFMA shadow. Sub-steps 0 .. KK-2 read the next sub-step's
        // fragments and carry this K step's global loads (for step kt + STAGES - 1, whose
        // buffer held step kt - 1); the last sub-step first waits for step kt + 1, meets
        // the other waves at the barrier and then reads step kt + 1's first fragments.
        // MORE: this step issues global loads; NEXT: a following K step exists. Both are
        // compile-time in each instance so the unrolled body has no branches.
        auto kstep = [&](int kt, auto more_c, auto next_c) {
            constexpr bool MORE = decltype(more_c)::value;
            constexpr bool NEXT = decltype(next_c)::value;
            const int lbuf = (kt + STAGES - 1) % STAGES, lk0 = (kt + STAGES - 1) * BK;
            const int cur = kt % STAGES;
            const int last_issued = min(kt + STAGES - 1, nk - 1);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const int fbuf = kk & 1;
                const bool last = kk == KK - 1;
                if (last && NEXT) {
                    wait_lgkm0();
                    wait_step(kt + 1, last_issued);
                    barrier_no_fence();
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < NMF; ++i) {
                    const int a = i / TN, b = i % TN;
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[fbuf][a], fb[fbuf][b], acc[a][b], 0, 0, 0);
                    if (i < NFR) {
                        if (!last) frag(fbuf ^ 1, cur, kk + 1, i);
                        else if (NEXT) frag(fbuf ^ 1, (kt + 1) % STAGES, 0, i);
                    }
                    if (MORE && !last && (i & 1) && (i >> 1) < LPS && kk * LPS + (i >> 1) < LOADS)
                        gload(lbuf, lk0, kk * LPS + (i >> 1));
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        int kt = 0;
        for (; kt + STAGES - 1 < nk; ++kt) kstep(kt, BoolC<true>{}, BoolC<true>{});
        for (; kt + 1 < nk; ++kt) kstep(kt, BoolC<false>{}, BoolC<true>{});
        if (kt < nk) kstep(kt, BoolC<false>{}, BoolC<false>{});
        __syncthreads();
    } else {
        u32x4 ra[Cfg::LA], rb[Cfg::LB];
#pragma unroll
        for (int p = 0; p < Cfg::LA; ++p) {
            const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
            ra[p] = *reinterpret_cast<const u32x4*>(Pt + row * ld + ch * 8);
        }
#pragma unroll
        for (int p = 0; p < Cfg::LB; ++p) {
            const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
            rb[p] = *reinterpret_cast<const u32x4*>(Qt + row * ld + ch * 8);
        }
#pragma unroll
        for (int p = 0; p < Cfg::LA; ++p) {
            const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
            *reinterpret_cast<u32x4*>(sA + gemm_swz<Cfg>(row, ch)) = ra[p];
        }
#pragma unroll
        for (int p = 0; p < Cfg::LB; ++p) {
            const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
            *reinterpret_cast<u32x4*>(sB + gemm_swz<Cfg>(row, ch)) = rb[p];
        }
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const bool more = kt + 1 < nk;
            if (more) {
                const int k0 = (kt + 1) * BK;
#pragma unroll
                for (int p = 0; p < Cfg::LA; ++p) {
                    const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
                    ra[p] = *reinterpret_cast<const u32x4*>(Pt + row * ld + k0 + ch * 8);
                }
#pragma unroll
                for (int p = 0; p < Cfg::LB; ++p) {
                    const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
                    rb[p] = *reinterpret_cast<const u32x4*>(Qt + row * ld + k0 + ch * 8);
                }
            }
            const unsigned short* a_s = sA + cur * STAGE_A;
            const unsigned short* b_s = sB + cur * STAGE_B;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                bf16x8 af[TM], bfr[TN];
                const int ch = kk * 2 + (lane >> 5);
#pragma unroll
                for (int a = 0; a < TM; ++a) {
                    const int row = wm * WM + a * 32 + (lane & 31);
                    af[a] = *reinterpret_cast<const bf16x8*>(a_s + gemm_swz<Cfg>(row, ch));
                }
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const int row = wn * WN + b * 32 + (lane & 31);
                    bfr[b] = *reinterpret_cast<const bf16x8*>(b_s + gemm_swz<Cfg>(row, ch));
                }
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int b = 0; b < TN; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
            }
            if (more) {
                unsigned short* an = sA + (cur ^ 1) * STAGE_A;
                unsigned short* bn = sB + (cur ^ 1) * STAGE_B;
#pragma unroll
                for (int p = 0; p < Cfg::LA; ++p) {
                    const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
                    *reinterpret_cast<u32x4*>(an + gemm_swz<Cfg>(row, ch)) = ra[p];
                }
#pragma unroll
                for (int p = 0; p < Cfg::LB; ++p) {
                    const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
                    *reinterpret_cast<u32x4*>(bn + gemm_swz<Cfg>(row, ch)) = rb[p];
                }
            }
            __syncthreads();
        }
    }

    // ---- epilogue. Accumulator element r of a 32x32 block sits at row
    // 8*(r/4) + 4*(lane/32) + r%4, column lane%32: each lane owns 4 consecutive rows of
    // one column, which are contiguous in the transposed layouts (X_c, the mirrored
    // half of A, W of a tall matrix). Every load of a block is issued before the
    // first use, so the epilogue pays one memory latency, not one per element group.
    const float first_s = args.first ? *d.scale : 1.0f;
    const int row_base = ti * BM + wm * WM;
    const int col_base = tj * BN + wn * WN;
    const int lj = lane & 31, li = (lane >> 5) * 4;

    if constexpr (MODE == kModeGram || MODE == kModePoly) {
        unsigned short* C = (MODE == kModeGram) ? d.a : d.b;
        const int64_t ldc = d.m_p;
        // b * A[i][j] with A symmetric: read A[j][i0 .. i0+3] (8 contiguous bytes); one
        // 32-row slab is prefetched ahead of the slab being stored
        u32x2 av[2][TN][4];
        auto load_a = [&](int buf, int a) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg)
                    av[buf][b][rg] = *reinterpret_cast<const u32x2*>(
                        d.a + (int64_t)(col_base + b * 32 + lj) * ldc + row_base + a * 32 + rg * 8 + li);
        };
        if constexpr (MODE == kModePoly) load_a(0, 0);
        const float g2 = first_s * first_s;
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            if constexpr (MODE == kModePoly) {
                if (a + 1 < TM) load_a((a + 1) & 1, a + 1);
            }
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int j = col_base + b * 32 + lj;
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int i0 = row_base + a * 32 + rg * 8 + li;
                    unsigned short h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x = acc[a][b][rg * 4 + e];
                        if constexpr (MODE == kModeGram) {
                            x *= g2;
                        } else {
                            const u32x2 w = av[a & 1][b][rg];
                            const unsigned w32 = (e < 2) ? w.x : w.y;
                            const float aij = bf2f((unsigned short)((e & 1) ? (w32 >> 16) : (w32 & 0xffff)));
                            x = fmaf(args.cb, aij, args.cc * x);
                        }
                        h[e] = f2bf(x);
                        C[(int64_t)(i0 + e) * ldc + j] = h[e];
                    }
                    if (ti != tj) {
                        u32x2 pk;
                        pk.x = pack2(h[0], h[1]);
                        pk.y = pack2(h[2], h[3]);
                        *reinterpret_cast<u32x2*>(C + (int64_t)j * ldc + i0) = pk;
                    }
                }
            }
        }
    } else {
        // a X[i][j] from X_c[j][i0 .. i0+3]; one 32-row slab is prefetched ahead
        u32x2 xv[2][TN][4];
        auto load_x = [&](int buf, int a) {
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg)
                    xv[buf][b][rg] = *reinterpret_cast<const u32x2*>(
                        d.xc + (int64_t)(col_base + b * 32 + lj) * d.m_p + row_base + a * 32 + rg * 8 + li);
        };
        load_x(0, 0);
#pragma unroll
        for (int a = 0; a < TM; ++a) {
            if (a + 1 < TM) load_x((a + 1) & 1, a + 1);
            // final modes: the W values of this 32-row slab are fetched before use
            float wv[TN][4][4];
            if constexpr (MODE == kModeFinalW) {
#pragma unroll
                for (int b = 0; b < TN; ++b) {
                    const int j = col_base + b * 32 + lj;
#pragma unroll
                    for (int rg = 0; rg < 4; ++rg) {
                        const int i0 = row_base + a * 32 + rg * 8 + li;
                        if (!d.tall) {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                wv[b][rg][e] = (i0 + e < d.m && j < d.n) ? d.out[(int64_t)(i0 + e) * d.n + j] : 0.f;
                        } else if (j < d.n && ((d.m & 3) == 0) && i0 + 3 < d.m) {
                            const floatx4 w4 = *reinterpret_cast<const floatx4*>(d.out + (int64_t)j * d.m + i0);
                            wv[b][rg][0] = w4.x; wv[b][rg][1] = w4.y; wv[b][rg][2] = w4.z; wv[b][rg][3] = w4.w;
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                wv[b][rg][e] = (i0 + e < d.m && j < d.n) ? d.out[(int64_t)j * d.m + i0 + e] : 0.f;
                        }
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int j = col_base + b * 32 + lj;
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int i0 = row_base + a * 32 + rg * 8 + li;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const u32x2 xw = xv[a & 1][b][rg];
                        const unsigned w32 = (e < 2) ? xw.x : xw.y;
                        const float x = bf2f((unsigned short)((e & 1) ? (w32 >> 16) : (w32 & 0xffff)));
                        v[e] = fmaf(args.ca, x, acc[a][b][rg * 4 + e]) * first_s;
                    }
                    if constexpr (MODE == kModeApply) {
                        unsigned short h[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            h[e] = f2bf(v[e]);
                            d.xr_next[(int64_t)(i0 + e) * d.n_p + j] = h[e];
                        }
                        u32x2 pk;
                        pk.x = pack2(h[0], h[1]);
                        pk.y = pack2(h[2], h[3]);
                        *reinterpret_cast<u32x2*>(d.xc_next + (int64_t)j * d.m_p + i0) = pk;
                    } else {
                        float r[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            if constexpr (MODE == kModeFinalO) r[e] = v[e];
                            else r[e] = fmaf(-d.upd_coef, v[e], wv[b][rg][e] * args.decay);
                        }
                        // O, or the Eq. 4 update of W, in the input orientation
                        if (!d.tall) {
                            if (j < d.n) {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (i0 + e < d.m) d.out[(int64_t)(i0 + e) * d.n + j] = r[e];
                            }
                        } else if (j < d.n) {
                            float* rowp = d.out + (int64_t)j * d.m;
                            if (((d.m & 3) == 0) && i0 + 3 < d.m) {
                                floatx4 o;
                                o.x = r[0]; o.y = r[1]; o.z = r[2]; o.w = r[3];
                                *reinterpret_cast<floatx4*>(rowp + i0) = o;
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (i0 + e < d.m) rowp[i0 + e] = r[e];
                            }
                        }
                    }
                }
            }
        }
    }
}

}  // namespace muon
