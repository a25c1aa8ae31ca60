// Newton-Schulz GEMM stage kernel template ("Muon is Scalable for LLM Training",
// Sec. 2.1 Eq. 2: X <- a X + b (X X^T) X + c (X X^T)^2 X).
//
// Each iteration is three products, all of the form C[i][j] = sum_k P[i][k] Q[j][k]:
//   Gram  A = X X^T            P = Q = X            K = n_p   symmetric output
//   Poly  P = aI + bA + cAA    P = Q = A            K = m_p   symmetric (A = A^T)
//   Apply X' = P X             P = P, Q = X_c       K = m_p   X'_c (and X'_r) out
// X_c = X^T ([n_p, m_p]), A and P ([m_p, m_p]) are panel-blocked in HBM (kb_off): a K
// step of a 256-row operand tile is one contiguous 16 KiB block. The big-tile Gram reads
// X_c as K-major tiles (rows k) and transposes in the fragment reads; the small-tile
// Gram reads the row-major copy X_r ([m_p, n_p]).
// X' = a X + (b A + c A^2) X is computed as (a I + b A + c A^2) X: the polynomial's
// epilogue adds a to the diagonal before its bf16 rounding, so the Apply is a plain
// product whose epilogue reads no operand. (Measured with a CPU emulation of the bf16
// rounding against the float64 iteration: this is also the more accurate recipe, since
// the diagonal a + B_ii that gets rounded is smaller than B_ii.)
// Symmetric outputs compute only upper-triangular tiles and store each tile twice
// (mirrored). The first iteration folds s = 1 / ||M||_F into the Gram (s^2) and
// Apply (s) epilogues. The last Apply writes fp32 O in the input's orientation, or
// applies Eq. 4 to W directly.
//
// Block: 256 threads = 2 x 2 waves, each wave a (BM/2) x (BN/2) sub-tile built from
// v_mfma_f32_32x32x16_bf16 blocks (fp32 accumulation).
//
// Big tiles (256 x 256, kDirect): K step 32 in a ring of 4 LDS stages, three K steps
// of loads in flight, one barrier per K step. The loads are buffer loads straight to
// LDS (buffer_load_dwordx4 ... lds): a resource over the tile's panel in scalar
// registers, one per-lane offset fixed for the whole K loop, a scalar offset per load;
// each lane's 16 bytes land at LDS base + 16 * lane, so lane l fetches the logical chunk
// that belongs at that (swizzled) position. The K loop is unrolled over the four ring
// stages, so every LDS offset is a constant, and it issues no vector-ALU instruction:
// measured on MI355X, vector-ALU work between MFMAs costs matrix-pipe throughput. K
// step 0 starts the accumulators from a zero accumulator input.
// Small tiles (128 x 128): K step 64 through registers (global -> VGPR -> LDS,
// ds_write_b128), double-buffered, loads for step k + 1 in flight while step k computes.
// K-contiguous LDS rows are swizzled: the 16-byte chunk c of row r sits at position
// c ^ ((r >> s) & (chunks per row - 1)), so the 16 rows that a 16-lane group reads land
// on distinct 16-byte bank groups (a plain (r & 7) swizzle left half of the LDS cycles
// in bank-conflict stalls).
//
// Tile order: consecutive blocks (which run together on one XCD after the remap)
// cover compact 2-D patches so that they share operand panels in L2: rectangular
// stages walk groups of 8 tile-rows column by column, symmetric stages walk 4 x 4
// super-tiles of the upper triangle.
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
    // epilogue staging, per wave and per half of its columns (HN of them): a bf16
    // transposed tile [HN][WM + 8] plus a bf16 direct tile [WM][HN + 8], or one fp32 tile
    static constexpr int HN = WN / 2;
    static constexpr int kEpiBf16 = (HN * (WM + 8) + WM * (HN + 8)) * 2;
    static constexpr int kEpiF32 = (HN * (WM + 4) > WM * (HN + 4) ? HN * (WM + 4) : WM * (HN + 4)) * 4;
    static constexpr int kEpiWave = ((kEpiBf16 > kEpiF32 ? kEpiBf16 : kEpiF32) + 15) / 16 * 16;
    static constexpr int kMainBytes = STAGES * (BM + BN) * BK * 2;
    // K-major operand tiles (rows k of BM = 256 columns, read with ds_read_b64_tr_b16):
    // a 1 KiB wave-wide load fills one slot with rows k and k + 4; slots are padded to
    // 1088 bytes; 16 slots hold the 32 rows of a K step.
    static constexpr bool kTrOK = kDirect && BK == 32 && BM == 256 && BN == 256;
    static constexpr int kTrSlot = 544;            // elements per slot (1024 + 64 bytes)
    static constexpr int kTrStage = 16 * kTrSlot;  // elements per operand per stage
    static constexpr int kMainBytesTr = kTrOK ? STAGES * 2 * kTrStage * 2 : 0;
    static constexpr int kMainMax = kMainBytes > kMainBytesTr ? kMainBytes : kMainBytesTr;
    static constexpr int kLdsBytes = kMainMax > 4 * kEpiWave ? kMainMax : 4 * kEpiWave;
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

// K-major tile: row k of a K step lives in slot (k & 3) + 4 (k >> 3), half (k >> 2) & 1
// (slot = 1 KiB load + 64 bytes of padding). The four rows k, k + 1, k + 2, k + 3 that
// one 32-lane half of a transposing read touches sit in four consecutive slots, i.e. in
// four different 64-byte bank windows, and every offset is a sum of a per-lane term
// and compile-time terms.
template <class Cfg>
__device__ __forceinline__ int tr_off(int k, int col) {
    return ((k & 3) + 4 * (k >> 3)) * Cfg::kTrSlot + ((k >> 2) & 1) * 256 + col;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16 on gfx950: within each group of 16 lanes, output lane 4q + r
// receives element r of the 8-byte chunks addressed by lanes q, q + 4, q + 8, q + 12
// (in that order): a 16 x 4 block of 16-bit values is transposed across the group.
__device__ __forceinline__ v4i16 lds_read_tr16(const unsigned short* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
}

template <bool B>
struct BoolC {
    static constexpr bool value = B;
};

template <int N>
struct IntC {
    static constexpr int value = N;
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

// Slot `sl` of XCD x -> (matrix gi, tile index local): every XCD walks the group's
// matrices in order and takes one contiguous eighth of each one's tiles, eighth
// (x + rot) & 7 of matrix g (the host picks rot to balance the XCDs). gi = -1 when the
// XCD has fewer slots.
__device__ __forceinline__ void xcd_slot(const NsArgs& args, int x, int sl, int& gi, int& local) {
    gi = -1;
    for (int g = 0; g < args.n; ++g) {
        const int T = args.d[g].ntiles, j = (x + args.d[g].rot) & 7;
        const int lo = (j * T) >> 3, cnt = (((j + 1) * T) >> 3) - lo;
        if (sl < cnt) {
            gi = g;
            local = lo + sl;
            return;
        }
        sl -= cnt;
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// kSplitOK: the instance used by launches that split their tail tiles (the others
// compile without the chunk logic).
template <int MODE, class Cfg, bool kSplitOK = false>
__device__ __forceinline__ void ns_gemm_tile(const NsArgs& args, unsigned short* smem) {
    constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, NT = Cfg::NT;
    constexpr int WM = Cfg::WM, WN = Cfg::WN, TM = Cfg::TM, TN = Cfg::TN;
    // The big Gram reads both operands from X_c ([n_p, m_p], K = n along its rows):
    // K-major tiles and transposing fragment reads. Every other stage reads K-contiguous
    // rows (the small Gram from X_r).
    constexpr bool kTr = (MODE == kModeGram) && Cfg::kTrOK;
    constexpr int STAGE_A = kTr ? Cfg::kTrStage : BM * BK, STAGE_B = kTr ? Cfg::kTrStage : BN * BK;
    unsigned short* const sA = smem;
    unsigned short* const sB = smem + Cfg::STAGES * STAGE_A;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Blocks are dealt round-robin over the 8 XCDs (block b runs on XCD b % 8). Every
    // XCD walks the group's matrices in order (longest K first) and takes one contiguous
    // eighth of each matrix's tile sequence, the eighths rotated per matrix to balance
    // the XCDs' work even when the matrices' K differ, and neighbouring tiles (shared
    // operand panels) in the same L2. Blocks left without a tile (the grid is 8 x the
    // largest per-XCD count) exit here.
    constexpr bool kSym = (MODE == kModeGram || MODE == kModePoly);
    // Split tiles (Gram, polynomial and non-final Apply on the direct-load tile): the
    // XCD's tiles xfull[x] .. xfull[x] + xtail[x] - 1 run as S = xsplit[x] chunks of K
    // each. Its blocks from xfull[x] on, u = block - xfull[x], are chunk u % S of tile
    // xfull[x] + u / S while u < xtail[x] S, then the tiles after the split ones, whole.
    // Tail split: the split tiles end the sequence. Head split: xfull[x] = 0.
    constexpr bool kSplit = (kSym || MODE == kModeApply) && Cfg::kDirect && kSplitOK;
    int chunk = -1, nsplit = 1, unit = 0;
    int gi = -1, local = 0;
    {
        const int x = blockIdx.x & 7;
        int sl = blockIdx.x >> 3;
        if constexpr (kSplit) {
            if (sl >= args.xfull[x]) {
                const int u = sl - args.xfull[x];
                const int nt = args.xtail[x], S = args.xsplit[x];
                if (u < nt * S) {
                    nsplit = S;
                    chunk = u % S;
                    sl = args.xfull[x] + u / S;
                    unit = args.xpbase[x] + u;
                } else {
                    sl = args.xfull[x] + nt + (u - nt * S);
                }
            }
        }
        xcd_slot(args, x, sl, gi, local);
    }
    if (gi < 0) return;
    const NsDesc d = args.d[gi];  // a copy: the kernel arguments are then read only at fixed or indexed offsets

    int ti, tj;
    if constexpr (kSym) tri_tile(local, d.tiles, ti, tj);
    else rect_tile(local, d.m_p / BM, d.tiles, ti, tj);

    const unsigned short* P;
    const unsigned short* Q;
    int64_t ld;
    int K;
    if constexpr (kTr) { P = d.xc; Q = d.xc; ld = d.m_p; K = d.n_p; }
    else if constexpr (MODE == kModeGram) { P = d.xr; Q = d.xr; ld = d.n_p; K = d.n_p; }
    else if constexpr (MODE == kModePoly) { P = d.a; Q = d.a; ld = d.m_p; K = d.m_p; }
    else { P = d.b; Q = d.xc; ld = d.m_p; K = d.m_p; }
    // X_c, A and B are panel-blocked (kb_off); only the small-tile Gram's X_r is row-major.
    // K-major tiles (kTr) start at the tile's first column block; the others at the
    // tile's first row.
    constexpr bool kBlk = kTr || MODE != kModeGram;
    const unsigned short* Pt;
    const unsigned short* Qt;
    if constexpr (kTr) {
        Pt = P + ((int64_t)ti * (BM / 32) << 13);
        Qt = Q + ((int64_t)tj * (BN / 32) << 13);
    } else if constexpr (kBlk) {
        Pt = P + kb_off((int64_t)ti * BM, 0, K);
        Qt = Q + kb_off((int64_t)tj * BN, 0, K);
    } else {
        Pt = P + (int64_t)ti * BM * ld;
        Qt = Q + (int64_t)tj * BN * ld;
    }

    // The direct-load path starts the accumulators with its first K step's MFMAs (a zero
    // accumulator input) instead of writing 16 zeros into each of them.
    floatx16 acc[TM][TN];
    if constexpr (!Cfg::kDirect) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int b = 0; b < TN; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    }

    // K steps of this block: all of K, or chunk c of nsplit, cut at multiples of 256 (K
    // is one): the chunk's start is then a fixed offset of the tile's operand pointers
    // in both the K-major and the K-contiguous panel layouts.
    int nk = K / BK;
    if (chunk >= 0) {
        const int n256 = K >> 8;
        const int c0 = (chunk * n256) / nsplit, c1 = ((chunk + 1) * n256) / nsplit;
        nk = (c1 - c0) * (256 / BK);
        const int64_t kofs = kTr ? (((int64_t)c0 * (ld >> 5)) << 13) : ((int64_t)(c0 * 8) << 13);
        Pt += kofs;
        Qt += kofs;
    }
    // partial tile of unit u, this wave's accumulators in register order (256-byte rows)
    float* const tail_w = kSplit ? args.tail + (int64_t)unit * kTailUnitFloats + wave * (TM * TN * 16 * 64) + lane
                                 : nullptr;

    if constexpr (Cfg::kDirect) {
        // 1 KiB load j covers rows RPI*j .. RPI*j + RPI-1: lane l lands on row
        // RPI*j + l / CPR at physical chunk l % CPR, so it fetches the logical chunk that
        // the swizzle stores there (the XOR is its own inverse).
        constexpr int STAGES = Cfg::STAGES, RPI = Cfg::RPI, CPR = Cfg::CPR;
        constexpr int LOADS = Cfg::IA + Cfg::IB;  // wave-wide loads per K step
        constexpr int KK = BK / 16;               // MFMA sub-steps per K step
        constexpr int NMF = TM * TN;              // MFMAs per sub-step
        // LDS reads per sub-step: one 16-byte read per fragment, or two transposing
        // 8-byte reads (k 0-3 and 4-7 of the lane's 8) for K-major tiles
        constexpr int NFR = kTr ? 2 * (TM + TN) : TM + TN;
        constexpr int LPS = (LOADS + KK - 2) / (KK - 1);  // global loads per sub-step
        static_assert(KK >= 2 && KK % 2 == 0, "sub-step parity must restart at 0 every K step");
        static_assert(NFR <= NMF && 2 * LPS <= NMF, "issue slots");
        static_assert(!kTr || (Cfg::IA == 4 && Cfg::IB == 4), "K-major tiles: 16 loads of two rows each");
        static_assert(kBlk && BK == 32 && BM == 256 && BN == 256, "a direct-load tile is one blocked panel, K step one block");
        // the wave index is uniform: keep it scalar so the LDS destinations (M0) are too
        const int swave = __builtin_amdgcn_readfirstlane(wave);
        const int lrow = lane / CPR, lpc = lane % CPR;
        // The loads are buffer loads to LDS: a resource over the tile's panel (scalar
        // registers), a per-lane byte offset that is the same for every load and K step
        // (vector), and a block-uniform byte offset per load and K step (scalar). No load
        // needs vector address arithmetic.
        // Load q of this wave covers slot (or 16-row group) swave * I + q:
        //   K-major tiles: lane l fetches 16-byte chunk (l & 31) of row 4 (l >> 5) of the
        //   slot's row pair, rows (s & 3) + 8 (s >> 2) (+ 4) of the K step's 32;
        //   K-contiguous tiles: lane l fetches row l / CPR of the group at the swizzled
        //   chunk position, and the swizzle depends on the lane alone (the group's first
        //   row is a multiple of RPI, which keeps (row >> SWS) mod CPR to the lane's part).
        static_assert(kTr || ((RPI >> Cfg::SWS) % CPR) == 0, "swizzle independent of the load index");
        uint32_t lane_off;  // bytes
        if constexpr (kTr) {
            const int c = lane & 31;
            lane_off = 2u * (((uint32_t)(c >> 2) << 13) + 4 * (lane >> 5) * 32 + ((c & 3) << 3));
        } else {
            lane_off = 2u * (uint32_t)(lrow * BK + ((lpc ^ ((lrow >> Cfg::SWS) & (CPR - 1))) << 3));
        }
        auto slot_off = [&](int sl) -> uint32_t {  // bytes, block-uniform
            if constexpr (kTr) return 2u * (uint32_t)(((sl & 3) + 8 * (sl >> 2)) * 32);
            else return 2u * (uint32_t)(sl * RPI * BK);
        };
        // the panel bases are block-uniform; reading them through readfirstlane tells the
        // compiler so (a resource it takes for per-lane data costs a loop per load)
        auto uniform_ptr = [](const unsigned short* q) -> void* {
            const uint64_t v = reinterpret_cast<uint64_t>(q);
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
            return reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
        };
        const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(Pt), (short)0, 0x7FFFFFFF, 0x00020000);
        const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(Qt), (short)0, 0x7FFFFFFF, 0x00020000);
        // one 1 KiB load (idx < LOADS) into the stage whose A and B tiles start at dA, dB
        auto gload = [&](unsigned short* dA, unsigned short* dB, int k0, int idx) {
            // K-major: rows k0 .. k0 + 31 of panel k0 / 256; otherwise block k0 / 32
            const uint32_t kofs = 2u * (uint32_t)(kTr ? ((((int64_t)(k0 >> 8) * (ld >> 5)) << 13) + ((k0 & 255) << 5))
                                                      : ((int64_t)(k0 >> 5) << 13));
            constexpr int SLOT = kTr ? Cfg::kTrSlot : 512;
            if (idx < Cfg::IA)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)(dA + (swave * Cfg::IA + idx) * SLOT), 16,
                                                         lane_off, kofs + slot_off(swave * Cfg::IA + idx), 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(dB + (swave * Cfg::IB + idx - Cfg::IA) * SLOT),
                                                         16, lane_off, kofs + slot_off(swave * Cfg::IB + idx - Cfg::IA), 0,
                                                         0);
        };
        // Fragments are double-buffered in registers (K-major tiles: as two halves).
        bf16x8 fa[2][TM], fb[2][TN];
        v4i16 fah[2][TM][2], fbh[2][TN][2];
        // one LDS read (r < NFR) of sub-step kk from the stage whose tiles start at cA, cB
        auto frag = [&](int fbuf, const unsigned short* cA, const unsigned short* cB, int kk, int r) {
            if constexpr (kTr) {
                // lane l addresses row k = 16 kk + 8 (l / 32) + 4 h + (l / 4) % 4 at column
                // 16 ((l / 16) % 2) + 4 (l % 4) of the fragment's 32 columns; after the
                // transposing read it holds column l % 32, k = 16 kk + 8 (l / 32) + 4 h + 0..3
                const int f = r >> 1, h = r & 1;
                const int k = kk * 16 + ((lane >> 5) << 3) + (h << 2) + ((lane >> 2) & 3);
                const int c = (((lane >> 4) & 1) << 4) + ((lane & 3) << 2);
                if (f < TM)
                    fah[fbuf][f][h] = lds_read_tr16(cA + tr_off<Cfg>(k, wm * WM + f * 32 + c));
                else
                    fbh[fbuf][f - TM][h] = lds_read_tr16(cB + tr_off<Cfg>(k, wn * WN + (f - TM) * 32 + c));
            } else {
                const int ch = kk * 2 + (lane >> 5);
                if (r < TM)
                    fa[fbuf][r] = *reinterpret_cast<const bf16x8*>(
                        cA + gemm_swz<Cfg>(wm * WM + r * 32 + (lane & 31), ch));
                else
                    fb[fbuf][r - TM] = *reinterpret_cast<const bf16x8*>(
                        cB + gemm_swz<Cfg>(wn * WN + (r - TM) * 32 + (lane & 31), ch));
            }
        };
        auto opa = [&](int fbuf, int a) -> bf16x8 {
            if constexpr (kTr)
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(fah[fbuf][a][0], fah[fbuf][a][1],
                                                                          0, 1, 2, 3, 4, 5, 6, 7));
            else
                return fa[fbuf][a];
        };
        auto opb = [&](int fbuf, int b) -> bf16x8 {
            if constexpr (kTr)
                return __builtin_bit_cast(bf16x8, __builtin_shufflevector(fbh[fbuf][b][0], fbh[fbuf][b][1],
                                                                          0, 1, 2, 3, 4, 5, 6, 7));
            else
                return fb[fbuf][b];
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
                for (int idx = 0; idx < LOADS; ++idx) gload(sA + st * STAGE_A, sB + st * STAGE_B, st * BK, idx);
        wait_step(0, min(STAGES - 2, nk - 1));
        barrier_no_fence();
#pragma unroll
        for (int r = 0; r < NFR; ++r) frag(0, sA, sB, 0, r);
        // Main loop. Each MFMA occupies the matrix pipe for 8 passes; the wave issues at
        // most one LDS read and one global load between two MFMAs, so the other issue
        // work hides in the MFMA shadow. Sub-steps 0 .. KK-2 read the next sub-step's
        // fragments and carry this K step's global loads (for step kt + STAGES - 1, whose
        // buffer held step kt - 1); the last sub-step first waits for step kt + 1, meets
        // the other waves at the barrier and then reads step kt + 1's first fragments.
        // MORE: this step issues global loads; NEXT: a following K step exists. Both are
        // compile-time in each instance so the unrolled body has no branches.
        //
        // The stage a K step loads into (kt + STAGES - 1) differs from the two it reads
        // (kt, kt + 1) when STAGES >= 3; passing the three stages as restrict pointers
        // tells the compiler so. Without it, a transposing LDS read after an LDS-DMA load
        // gets a wait for every outstanding load; the explicit waits above already order
        // each read after the loads of its own stage.
        static_assert(STAGES >= 3, "the load stage must differ from the stages read");
        // phase_c: IntC<p> when kt % STAGES == p is known at compile time (the stage
        // offsets then fold into the LDS instructions' immediate offsets), IntC<-1> when not.
        auto kstep = [&](int kt, auto more_c, auto next_c, auto phase_c, auto first_c) {
            constexpr bool MORE = decltype(more_c)::value;
            constexpr bool NEXT = decltype(next_c)::value;
            constexpr int PH = decltype(phase_c)::value;
            constexpr bool FIRST = decltype(first_c)::value;  // K step 0: accumulators start at zero
            const int lk0 = (kt + STAGES - 1) * BK;
            const int lbuf = PH >= 0 ? (PH + STAGES - 1) % STAGES : (kt + STAGES - 1) % STAGES;
            const int cur = PH >= 0 ? PH : kt % STAGES;
            const int nxt = PH >= 0 ? (PH + 1) % STAGES : (kt + 1) % STAGES;
            const int last_issued = min(kt + STAGES - 1, nk - 1);
            auto body = [&](unsigned short* __restrict__ dA, unsigned short* __restrict__ dB,
                            const unsigned short* __restrict__ cA, const unsigned short* __restrict__ cB,
                            const unsigned short* __restrict__ nA, const unsigned short* __restrict__ nB) {
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const int fbuf = kk & 1;
                    const bool last = kk == KK - 1;
                    if (last && NEXT) {
                        wait_lgkm0();
                        // a step that issues loads has issued STAGES - 2 steps beyond kt + 1
                        if constexpr (MORE) wait_vmcnt<LOADS * (STAGES - 2)>();
                        else wait_step(kt + 1, last_issued);
                        barrier_no_fence();
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < NMF; ++i) {
                        // snake order over the fragment grid: consecutive MFMAs differ in one
                        // operand only (fewer operand bits toggle; 0.2-0.3% faster, same sums)
                        const int a = i / TN, b = (a & 1) ? (TN - 1 - i % TN) : (i % TN);
                        if constexpr (FIRST) {
                            if (kk == 0) {
                                const floatx16 zero = {};
                                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa(fbuf, a), opb(fbuf, b), zero,
                                                                                   0, 0, 0);
                            } else {
                                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa(fbuf, a), opb(fbuf, b),
                                                                                   acc[a][b], 0, 0, 0);
                            }
                        } else {
                            acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa(fbuf, a), opb(fbuf, b), acc[a][b],
                                                                               0, 0, 0);
                        }
                        if (i < NFR) {
                            if (!last) frag(fbuf ^ 1, cA, cB, kk + 1, i);
                            else if (NEXT) frag(fbuf ^ 1, nA, nB, 0, i);
                        }
                        if (MORE && !last && (i & 1) && (i >> 1) < LPS && kk * LPS + (i >> 1) < LOADS)
                            gload(dA, dB, lk0, kk * LPS + (i >> 1));
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            };
            body(sA + lbuf * STAGE_A, sB + lbuf * STAGE_B, sA + cur * STAGE_A, sB + cur * STAGE_B,
                 sA + nxt * STAGE_A, sB + nxt * STAGE_B);
        };
        // The steps that issue loads run unrolled by the ring depth, so that every stage
        // offset is a constant; the few steps after them (at most STAGES - 1 that still
        // issue loads, then the STAGES - 1 that drain the ring) compute their stages.
        // K step 0 (which issues loads: K is at least one 256-wide unit, 8 steps) runs
        // first, on its own, with zero accumulator inputs.
        static_assert(STAGES == 4, "the unrolled K loop has four phases");
        constexpr BoolC<true> T{};
        constexpr BoolC<false> F{};
        kstep(0, T, T, IntC<0>{}, T);
        int kt = 1;
        for (; kt + STAGES - 1 + 3 < nk; kt += 4) {
            kstep(kt, T, T, IntC<1>{}, F);
            kstep(kt + 1, T, T, IntC<2>{}, F);
            kstep(kt + 2, T, T, IntC<3>{}, F);
            kstep(kt + 3, T, T, IntC<0>{}, F);
        }
        for (; kt + STAGES - 1 < nk; ++kt) kstep(kt, T, T, IntC<-1>{}, F);
        for (; kt + 1 < nk; ++kt) kstep(kt, F, T, IntC<-1>{}, F);
        if (kt < nk) kstep(kt, F, F, IntC<-1>{}, F);
        __syncthreads();
        if constexpr (kSplit) {
            if (chunk >= 0) {  // a tail chunk: partial sums out, the fixup finishes the tile
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int b = 0; b < TN; ++b)
#pragma unroll
                        for (int r = 0; r < 16; ++r) tail_w[((a * TN + b) * 16 + r) * 64] = acc[a][b][r];
                return;
            }
        }
    } else {
        // element (row, k) of the P / Q tile: blocked work matrices or the row-major X_r
        auto pa = [&](int row, int k) -> const unsigned short* {
            if constexpr (kBlk) return P + kb_off((int64_t)ti * BM + row, k, K);
            else return Pt + (int64_t)row * ld + k;
        };
        auto qa = [&](int row, int k) -> const unsigned short* {
            if constexpr (kBlk) return Q + kb_off((int64_t)tj * BN + row, k, K);
            else return Qt + (int64_t)row * ld + k;
        };
        u32x4 ra[Cfg::LA], rb[Cfg::LB];
#pragma unroll
        for (int p = 0; p < Cfg::LA; ++p) {
            const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
            ra[p] = *reinterpret_cast<const u32x4*>(pa(row, ch * 8));
        }
#pragma unroll
        for (int p = 0; p < Cfg::LB; ++p) {
            const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
            rb[p] = *reinterpret_cast<const u32x4*>(qa(row, ch * 8));
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
                    ra[p] = *reinterpret_cast<const u32x4*>(pa(row, k0 + ch * 8));
                }
#pragma unroll
                for (int p = 0; p < Cfg::LB; ++p) {
                    const int c = p * NT + tid, row = c / Cfg::CPR, ch = c % Cfg::CPR;
                    rb[p] = *reinterpret_cast<const u32x4*>(qa(row, k0 + ch * 8));
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
                    for (int bi = 0; bi < TN; ++bi) {
                        const int b = (a & 1) ? TN - 1 - bi : bi;  // snake order, as in the direct-load loop
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
                    }
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
    // one column. Results are staged per wave through LDS, a chunk of the wave's columns at
    // a time, and leave in 16-byte row chunks: the direct orientation C[i][j] and/or the
    // transposed one C[j][i] (X'_r / X'_c, a symmetric tile and its mirror, or W of a
    // flat / tall matrix). Operands of the epilogue math (the mirrored half
    // of A for b A) are read where a lane's 4 rows are contiguous.
    // The wave's columns leave in NCH chunks of HN: halves, or quarters for the fused
    // update, whose W loads for the next quarter are issued while the current one is
    // staged and stored (two quarters of W fit the registers, two halves do not).
    constexpr int NCH = (MODE == kModeFinalW && TN >= 4) ? 4 : 2;
    constexpr int HN = WN / NCH, NBH = TN / NCH;   // columns and 32-column blocks per chunk
    static_assert(NBH >= 1 && NBH * NCH == TN, "whole 32-column blocks per chunk");
    static_assert(HN <= Cfg::HN, "a chunk fits the staging area");
    constexpr int kWN = WM * HN / 4 / 64;          // fused update: W float4 per lane and chunk
    constexpr int TSB = WM + 8, DSB = HN + 8;     // bf16 strides: transposed, direct
    constexpr int TSF = WM + 4, DSF = HN + 4;     // fp32 strides
    const float first_s = args.first ? *d.scale : 1.0f;
    const int row_base = ti * BM + wm * WM;
    const int col_base = tj * BN + wn * WN;
    const int lj = lane & 31, li = (lane >> 5) * 4;
    unsigned short* const lt = sA + wave * (Cfg::kEpiWave / 2);   // transposed staging
    unsigned short* const ldr = lt + HN * TSB;                      // direct staging
    float* const lf = reinterpret_cast<float*>(lt);                 // fp32 staging

    constexpr bool kBf16Out = (MODE == kModeGram || MODE == kModePoly || MODE == kModeApply);
    // outputs of the bf16 modes
    unsigned short* dst_d = nullptr;  // direct [i][j]
    unsigned short* dst_t = nullptr;  // transposed [j][i]
    int64_t ld_d = 0, ld_t = 0;
    if constexpr (MODE == kModeGram || MODE == kModePoly) {
        dst_d = (MODE == kModeGram) ? d.a : d.b;
        dst_t = (ti != tj) ? dst_d : nullptr;
        ld_d = ld_t = d.m_p;
    } else if constexpr (MODE == kModeApply) {
        dst_d = d.xr_next;
        dst_t = d.xc_next;
        ld_d = d.n_p;
        ld_t = d.m_p;
    }
    const float g2 = first_s * first_s;
    float sq = 0.f;  // final modes: this lane's sum of O^2 (padding contributes exact zeros)

    // Operand of the polynomial's epilogue math (the mirrored half of A for b A), per
    // half: HN rows j of WM values i, 256 bytes each, brought in through LDS so that every
    // global access is a full 256-byte row segment (16 lanes per row, 4 rows per 1 KiB DMA
    // load) instead of 32 rows x 8 bytes per instruction. Chunk c of row r is stored at
    // position c ^ (r & 15). The block sits over the direct-staging area: it is read into
    // registers before any staging write, and x_dma waits until earlier LDS reads of the
    // area are done. The Apply stages read no operand here: the polynomial stage has
    // folded a I into P, so their epilogue only scales the product.
    constexpr bool kDmaX = MODE == kModePoly && Cfg::kDirect && WM == 128 && HN == 64;
    unsigned short* const xs = sA + __builtin_amdgcn_readfirstlane(wave) * (Cfg::kEpiWave / 2) + HN * TSB;
    auto x_dma = [&](int hh) {
        const unsigned short* src = d.a;
        const int64_t lds = d.m_p;
        wait_lgkm0();
        const int lr = lane >> 4, lp = lane & 15;
        const int j0 = col_base + hh * HN;
#pragma unroll
        for (int q = 0; q < HN / 4; ++q) {
            const int r = 4 * q + lr;
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src + kb_off(j0 + r, row_base + ((lp ^ (r & 15)) << 3), lds)),
                                             (lds_ptr_t)(xs + q * 512), 16, 0, 0);
        }
    };
    auto x_read = [&](u32x2 (&ov)[TM][NBH][4]) {
#pragma unroll
        for (int a = 0; a < TM; ++a)
#pragma unroll
            for (int bb = 0; bb < NBH; ++bb)
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int jl = bb * 32 + lj, ch = a * 4 + rg;
                    ov[a][bb][rg] = *reinterpret_cast<const u32x2*>(xs + jl * WM + ((ch ^ (jl & 15)) << 3) + li);
                }
    };

    // Fused update: W of chunk h as kWN float4 per lane. A tall W is [n, m] (row j holds
    // WM consecutive i of the tile), a flat one [m, n] (row i holds HN consecutive j of
    // the chunk).
    floatx4 wbuf[2][kWN];
    auto load_w = [&](floatx4 (&wv)[kWN], int hh) {
        const int colh0 = col_base + hh * HN;
        if (d.tall) {
            constexpr int CH = WM / 4;
#pragma unroll
            for (int it = 0; it < kWN; ++it) {
                const int c = it * 64 + lane, r = c / CH, k = c % CH;
                const int j = colh0 + r, i = row_base + k * 4;
                if (j < d.n && ((d.m & 3) == 0) && i + 3 < d.m)
                    wv[it] = *reinterpret_cast<const floatx4*>(d.out + (int64_t)j * d.m + i);
                else
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wv[it][e] = (j < d.n && i + e < d.m) ? d.out[(int64_t)j * d.m + i + e] : 0.f;
            }
        } else {
            constexpr int CH = HN / 4;
#pragma unroll
            for (int it = 0; it < kWN; ++it) {
                const int c = it * 64 + lane, r = c / CH, k = c % CH;
                const int i = row_base + r, j = colh0 + k * 4;
                if (i < d.m && ((d.n & 3) == 0) && j + 3 < d.n)
                    wv[it] = *reinterpret_cast<const floatx4*>(d.out + (int64_t)i * d.n + j);
                else
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        wv[it][e] = (i < d.m && j + e < d.n) ? d.out[(int64_t)i * d.n + j + e] : 0.f;
            }
        }
    };
    if constexpr (MODE == kModeFinalW) load_w(wbuf[0], 0);

#pragma unroll
    for (int h = 0; h < NCH; ++h) {
        // A chunk's work stays inside the chunk, apart from the next chunk's W loads,
        // which are issued here so that they overlap this chunk's staging and stores.
        __builtin_amdgcn_sched_barrier(0);
        const int colh0 = col_base + h * HN;  // first global column of this chunk
        if constexpr (MODE == kModeFinalW) {
            if (h + 1 < NCH) load_w(wbuf[(h + 1) & 1], h + 1);
        }
        // operands of the polynomial's epilogue math for this chunk: 8 contiguous bytes
        // per (a, b, rg)
        u32x2 opv[TM][NBH][4];
        if constexpr (MODE == kModePoly) {
            if (kDmaX) {
                x_dma(h);
                wait_vmcnt<0>();
                x_read(opv);
            } else {
                const unsigned short* src = d.a;
                const int64_t lds = d.m_p;  // A is [m_p, m_p]
#pragma unroll
                for (int a = 0; a < TM; ++a)
#pragma unroll
                    for (int bb = 0; bb < NBH; ++bb)
#pragma unroll
                        for (int rg = 0; rg < 4; ++rg)
                            opv[a][bb][rg] = *reinterpret_cast<const u32x2*>(
                                src + kb_off(col_base + (h * NBH + bb) * 32 + lj, row_base + a * 32 + rg * 8 + li, lds));
            }
        }
        // values -> LDS
#pragma unroll
        for (int a = 0; a < TM; ++a) {
#pragma unroll
            for (int bb = 0; bb < NBH; ++bb) {
                const int b = h * NBH + bb;
                const int jl = bb * 32 + lj;  // column within the chunk
#pragma unroll
                for (int rg = 0; rg < 4; ++rg) {
                    const int il = a * 32 + rg * 8 + li;  // first of 4 rows within the wave tile
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x = acc[a][b][rg * 4 + e];
                        if constexpr (MODE == kModeGram) {
                            x *= g2;
                        } else if constexpr (MODE == kModePoly) {
                            const u32x2 w = opv[a][bb][rg];
                            const unsigned w32 = (e < 2) ? w.x : w.y;
                            const float o = bf2f((unsigned short)((e & 1) ? (w32 >> 16) : (w32 & 0xffff)));
                            x = fmaf(args.cb, o, args.cc * x);
                            // P = a I + b A + c A A: a on the diagonal of the real rows
                            const int gi = row_base + il + e;
                            if (ti == tj && gi == colh0 + jl && gi < d.m) x += args.ca;
                        } else {
                            x *= first_s;  // P X, and s on the first iteration
                        }
                        v[e] = x;
                        if constexpr (!kBf16Out) sq = fmaf(x, x, sq);
                    }
                    if constexpr (kBf16Out) {
                        unsigned short hv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) hv[e] = f2bf(v[e]);
                        u32x2 pk;
                        pk.x = pack2(hv[0], hv[1]);
                        pk.y = pack2(hv[2], hv[3]);
                        *reinterpret_cast<u32x2*>(lt + jl * TSB + il) = pk;
                        if (dst_d) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) ldr[(il + e) * DSB + jl] = hv[e];
                        }
                    } else if (d.tall) {
                        floatx4 o;
                        o.x = v[0]; o.y = v[1]; o.z = v[2]; o.w = v[3];
                        *reinterpret_cast<floatx4*>(lf + jl * TSF + il) = o;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) lf[(il + e) * DSF + jl] = v[e];
                    }
                }
            }
        }
        wait_lgkm0();  // this wave's staging writes are complete before its lanes read them
        const int colh = colh0;
        if constexpr (kBf16Out) {
            // transposed rows: HN rows of WM values (WM / 8 chunks each)
            if (dst_t) {
#pragma unroll
                for (int it = 0; it < HN * WM / 8 / 64; ++it) {
                    const int c = it * 64 + lane, r = c / (WM / 8), k = c % (WM / 8);
                    const u32x4 val = *reinterpret_cast<const u32x4*>(lt + r * TSB + k * 8);
                    // non-temporal: the outputs are read by the next launch, not by this
                    // one, and kept out of the way of the operand slices in L2
                    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst_t + kb_off(colh + r, row_base + k * 8, ld_t)));
                }
            }
            // direct rows: WM rows of HN values (HN / 8 chunks each); X'_r only when the
            // next Gram runs on small tiles
            if (dst_d) {
#pragma unroll
                for (int it = 0; it < WM * HN / 8 / 64; ++it) {
                    const int c = it * 64 + lane, r = c / (HN / 8), k = c % (HN / 8);
                    const u32x4 val = *reinterpret_cast<const u32x4*>(ldr + r * DSB + k * 8);
                    // A and B are blocked; the Apply's X'_r is row-major
                    const int64_t o = (MODE == kModeApply) ? (int64_t)(row_base + r) * ld_d + colh + k * 8
                                                           : kb_off(row_base + r, colh + k * 8, ld_d);
                    __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(dst_d + o));
                }
            }
        } else if (d.tall) {
            // O / W is [n, m]: row j holds WM consecutive i of this tile (WM / 4 chunks)
            constexpr int CH = WM / 4, N = HN * CH / 64;
            static_assert(N == kWN, "W staging");
#pragma unroll
            for (int it = 0; it < N; ++it) {
                if (it % 8 == 0) __builtin_amdgcn_sched_barrier(0);  // at most 8 LDS reads ahead
                const int c = it * 64 + lane, r = c / CH, k = c % CH;
                const int j = colh + r, i = row_base + k * 4;
                floatx4 o = *reinterpret_cast<const floatx4*>(lf + r * TSF + k * 4);
                if constexpr (MODE == kModeFinalW) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = fmaf(-d.upd_coef, o[e], wbuf[h & 1][it][e] * args.decay);
                }
                if (j < d.n && ((d.m & 3) == 0) && i + 3 < d.m) {
                    *reinterpret_cast<floatx4*>(d.out + (int64_t)j * d.m + i) = o;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (j < d.n && i + e < d.m) d.out[(int64_t)j * d.m + i + e] = o[e];
                }
            }
        } else {
            // O / W is [m, n]: row i holds HN consecutive j of this chunk (HN / 4 float4)
            constexpr int CH = HN / 4, N = WM * CH / 64;
            static_assert(N == kWN, "W staging");
#pragma unroll
            for (int it = 0; it < N; ++it) {
                if (it % 8 == 0) __builtin_amdgcn_sched_barrier(0);  // at most 8 LDS reads ahead
                const int c = it * 64 + lane, r = c / CH, k = c % CH;
                const int i = row_base + r, j = colh + k * 4;
                floatx4 o = *reinterpret_cast<const floatx4*>(lf + r * DSF + k * 4);
                if constexpr (MODE == kModeFinalW) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = fmaf(-d.upd_coef, o[e], wbuf[h & 1][it][e] * args.decay);
                }
                if (i < d.m && ((d.n & 3) == 0) && j + 3 < d.n) {
                    *reinterpret_cast<floatx4*>(d.out + (int64_t)i * d.n + j) = o;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (i < d.m && j + e < d.n) d.out[(int64_t)i * d.n + j + e] = o[e];
                }
            }
        }
        // the next chunk overwrites the staging area: LDS executes a wave's operations in
        // order, so its writes cannot overtake the reads above
    }
    if constexpr (!kBf16Out) {
        static_assert(NT == 256, "four per-wave partials per tile");
        if (d.part) {
            const float t = wave_sum(sq);
            if (lane == 0) d.part[local * 4 + wave] = t;
        }
    }
}

}  // namespace muon
