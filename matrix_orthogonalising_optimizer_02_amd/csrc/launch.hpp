// Kernel descriptors and host-side launchers (internal to libmuon_rocm.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace muon {

// ---- momentum + Frobenius partials + bf16 working copies ------------------------
// One 64x64 tile per block over the padded [rows_p, cols_p] extent of M [rows, cols].
// `direct` receives bf16(M') in M's orientation ([rows_p, cols_p]); `transp` the
// transpose ([cols_p, rows_p]). Flat matrices: direct = X_r, transp = X_c; tall
// matrices: direct = X_c, transp = X_r. Padding is written as zeros. A null `direct`
// or `transp` is skipped (X_r is written only for groups whose Gram uses small tiles).
// X_c is panel-blocked (see kb_off), X_r row-major.
struct CastDesc {
    const float* m_in;
    const float* g;        // unused when the launch has use_momentum == 0
    float* m_out;          // M' written here when non-null (may equal m_in)
    unsigned short* direct;
    unsigned short* transp;
    float* partial;        // one float per tile: sum of M'^2 over the tile
    int32_t direct_blk;    // nonzero: `direct` is panel-blocked (kb_off), else row-major
    int32_t transp_blk;    // the same for `transp`
    int32_t rows, cols, rows_p, cols_p;
    int32_t tiles_c;       // cols_p / 64
    int32_t tile_begin;    // first tile of this matrix in the launch
    int32_t wide;          // nonzero: no transposed copy; tiles of 16 rows x 256 columns
};

struct CastArgs {
    CastDesc d[kMaxGroup];
    int32_t n;
    int32_t total;
    float mu;
    int32_t use_momentum;
};

// ---- per-matrix 1 / max(||M||_F, eps) from the tile partials -------------------
struct FrobArgs {
    const float* partial[kMaxGroup];
    float* scale[kMaxGroup];
    int32_t count[kMaxGroup];
    int32_t n;
    float eps;
};

// ---- NS5 GEMM stages (bf16 MFMA, fp32 accumulation) ----------------------------
// Working matrix X is [m, n] with m = min(rows, cols), n = max(rows, cols), padded
// to [m_p, n_p]. X_r is X row-major [m_p, n_p]; X_c is X^T row-major [n_p, m_p].
enum GemmMode : int {
    kModeGram = 0,     // A = s2 * X X^T                  (symmetric tiles)
    kModePoly = 1,     // P = a I + b A + c A A            (symmetric tiles; a on real rows only)
    kModeApply = 2,    // X' = s1 * P X                    bf16 X'_c, and X'_r if xr_next
    kModeFinalO = 3,   // O  = s1 * P X                    fp32, input orientation
    kModeFinalW = 4,   // W <- decay W - upd_coef O        fused Eq. 4 update
};

struct NsDesc {
    const unsigned short* xr;
    const unsigned short* xc;
    unsigned short* xr_next;
    unsigned short* xc_next;
    unsigned short* a;
    unsigned short* b;
    float* out;            // O or W: [rows, cols] row-major in the input orientation
    const float* scale;    // device scalar s = 1 / max(||M||_F, eps)
    int32_t m, n, m_p, n_p;
    int32_t tall;
    int32_t ntiles;        // tiles of this matrix in the stage
    int32_t tiles;         // symmetric: tiles per side; rectangular: tiles along n
    int32_t rot;           // XCD x takes eighth (x + rot) & 7 of this matrix's tiles
    float upd_coef;        // lr * (the update's direction scale), fused Eq. 4 / 5 update
    float* part;           // final modes, optional: [ntiles * 4] per-wave sums of O^2
};

// Gram, polynomial and non-final Apply stages on big tiles may split tiles of an XCD in
// K: tiles xfull[x] .. xfull[x] + xtail[x] - 1 of its sequence run as xsplit[x] chunks
// of K each (blocks xfull[x] .. xfull[x] + xtail[x] * xsplit[x] - 1 of the XCD; any
// tiles after them follow, whole), writing fp32 partial tiles (kTailUnitFloats each,
// accumulator order) at tail + (xpbase[x] + u) * kTailUnitFloats. The tail split takes
// the last round's tiles; the head split (xfull[x] = 0) the first, longest tiles of a
// one-round stage with mixed K. A fixup launch of sum(xtail) tiles adds each tile's
// chunks in chunk order and runs the stage's epilogue. tail == nullptr: no split.
#ifndef MUON_GEMM_TAIL_SPLIT
#define MUON_GEMM_TAIL_SPLIT 1
#endif
constexpr bool kGemmTailSplit = MUON_GEMM_TAIL_SPLIT != 0;
constexpr int kTailUnitFloats = 256 * 256;
constexpr int kTailMaxSplit = 8;
struct NsArgs {
    NsDesc d[kMaxGroup];
    int32_t n;
    int32_t total;         // grid size: 8 x the largest per-XCD block count
    float ca, cb, cc;
    float decay;           // 1 - lr * weight_decay
    int32_t first;         // first iteration: fold s into the epilogues
    float* tail;
    int32_t xfull[8], xtail[8], xsplit[8], xpbase[8];
    int32_t fix_total;     // blocks of the fixup launch
};

// ---- RowNorm step ---------------------------------------------------------------
struct RowDesc {
    const float* g;
    float* m;
    float* w;
    int32_t rows, cols;
    int32_t row_begin;     // first block of this matrix in the launch
    float coef;            // lr * gamma * (the update's direction scale)
    float* part;           // optional: [rows] sums of R^2 per row
};

struct RowArgs {
    RowDesc d[kMaxGroup];
    int32_t n;
    int32_t total;
    float mu, decay, eps;
};

struct ColDesc {
    const float* g;
    float* m;
    float* w;
    float* partial;        // [chunks, cols] per-chunk column sums of M'^2
    float* inv;            // [cols] 1 / max(column norm, eps)
    int32_t rows, cols;
    int32_t chunks;        // ceil(rows / kColChunkRows)
    int32_t tiles_c;       // ceil(cols / 256)
    int32_t tile_begin;    // first block of this matrix in the launch
    int32_t fin_begin;     // first block of this matrix in the finalize launch (kColFinCols columns each)
    float coef;
    float* part;           // optional: [cols] sums of R^2 per column
};

struct ColArgs {
    ColDesc d[kMaxGroup];
    int32_t n;
    int32_t total;
    float mu, decay, eps;
    int32_t sums_only;     // finalize: write the raw column sums of squares into `inv`
};

// ---- update RMS and the Eq. 6 scale -------------------------------------------
// One block per matrix sums `count` partial sums of U^2 (fixed order, double) into
// RMS(U) = sqrt(sum / elems). Eq. 6 refresh (eq6 != 0): coef_out = lr * rms_scale /
// max(RMS(O), eps) and the monitor reads rms_scale * RMS(O) / max(RMS(O), eps).
// Otherwise the monitor reads dir_scale * RMS(U).
struct RmsDesc {
    const float* part;
    float* coef_out;       // eq6: device scalar for the update kernel
    float* rms_out;        // optional: the caller's monitor entry
    double elems;          // rows * cols
    float dir_scale;
    int32_t count;
    int32_t eq6;
};

struct RmsArgs {
    RmsDesc d[kMaxGroup];
    int32_t n;
    float lr, rms_scale, eps;
};

// W <- decay W - coef O over [rows, cols] (O fp32, same layout as W); 4096 elements
// per block.
struct UpdDesc {
    const float* o;
    float* w;
    const float* coef;     // device scalar
    int64_t elems;
    int32_t blk_begin;
};

struct UpdArgs {
    UpdDesc d[kMaxGroup];
    int32_t n;
    int32_t total;
    float decay;
};

constexpr int kUpdBlockElems = 4096;

// ---- AdamW for the hybrid optimizer's non-matrix parameters ---------------------
// Tensors of any shape as flat fp32 arrays; 4096 elements per block; descriptors of
// up to kAdamMaxTensors tensors travel in the kernel arguments.
struct AdamDesc {
    float* w;
    float* m;
    float* v;
    const float* g;
    int64_t n;
    int32_t blk_begin;     // first block of this tensor in the launch
    int32_t pad_;
};

constexpr int kAdamMaxTensors = 48;
constexpr int kAdamBlockElems = 4096;

struct AdamArgs {
    AdamDesc d[kAdamMaxTensors];
    int32_t n;
    int32_t total;
    float beta1, beta2, one_minus_beta1, one_minus_beta2;
    float eps;
    float decay;           // 1 - lr * weight_decay
    float lr_bc1;          // lr / (1 - beta1^t)
    float inv_sqrt_bc2;    // 1 / sqrt(1 - beta2^t)
};

// ---- singular-spectrum diagnostic (SVD entropy), fp64 throughout -------------------
// For X = W (rows <= cols) or W^T (rows > cols), [m, n], the eigenvalues of the Gram
// matrix S = X X^T are sigma_i^2. S (m_p x m_p, m_p = m rounded up to kSpTile, zero
// padding) is reduced to tridiagonal form by Householder reflections, one column per
// step: step j's house kernel forms reflector v_j from row j (after the previous step's
// rank-2 update, applied on the fly); the pass kernel applies that update to the upper
// triangle of the trailing block, tile by tile, and leaves per-tile row and column sums
// of A v_j, which the reduce kernel adds in a fixed order into p_j = tau_j A v_j. Only
// the upper triangle is kept current (the lower one is stale after step 0). The
// eigenvalues of the tridiagonal matrix come from Sturm-count bisection.
constexpr int kSpTile = 128;        // Gram block tile (4 waves of 64 x 64)
constexpr int kSpPassTile = 64;     // pass kernel tile (upper-triangle tiles of the trailing block)
constexpr int kSpBisectIters = 80;  // bound on bisection halvings (stops earlier)

struct SpDesc {
    const float* w;        // [rows, cols] fp32 row-major input
    int64_t cols;          // leading dimension of w
    int32_t m, n;          // working dims: m = min(rows, cols), n = max
    int32_t tall;          // rows > cols: X = W^T
    int32_t tm;            // Gram tiles per side, ceil(m / kSpTile)
    int32_t tile_begin;    // first Gram tile of this matrix in the launch
    int64_t sigma_off;     // offset of this matrix's values in sigma_sq (if any)
    int64_t ld;            // leading dimension of s (m_p)
    double* s;             // symmetric work matrix, m_p x m_p
    double* v[2];          // Householder vectors v_j in v[j & 1] (entries j+1 .. m-1)
    double* wv;            // w_{j-1} = p_{j-1} - (tau_{j-1} / 2) (p_{j-1} . v_{j-1}) v_{j-1}
    double* p;             // p_j = tau_j S^(j) v_j
    double* rowpart;       // pass partials [tp][tp][64]: tile (I, J) row sums of A v
    double* colpart;       // pass partials [tp][tp][64]: tile (I, J) column sums (mirror)
    int32_t tp;            // partial-array tile dimension, m_p / kSpPassTile
    double* d;             // tridiagonal: diagonal (m)
    double* e;             // tridiagonal: sub-diagonal (m - 1)
    double* lam;           // eigenvalues, ascending (m)
    double* tau;           // tau_j in tau[j & 1]
    double* entropy;       // output: one value
};

struct SpArgs {
    SpDesc d[kMaxGroup];
    int32_t n;
    int32_t total;         // Gram: total tiles of the launch
    int32_t j;             // house / pass: the column step
    double* sigma_sq;      // optional output, descending per matrix (null = not wanted)
};

// Tall RowNorm blocks: kColChunkRows rows x kColTileCols columns, one partial row of
// column sums per chunk. 64-row blocks that each load their rows in one batch stream at
// 6.2 TB/s on MI355X against 5.5 TB/s for 256-row blocks that loop over four batches
// (the same read-read-write pattern on a [30720, 5120] matrix).
constexpr int kColChunkRows = 64;
constexpr int kColTileCols = 256;
// Columns per block of the finalize, which adds a column's chunk partials.
constexpr int kColFinCols = 64;
// Rows up to this length keep M' in registers (one 256-thread block per row; rows
// longer than kRowWideCols whose length is a multiple of 4 take a 1024-thread block).
constexpr int kRowMaxRegisterCols = 32 * 1024;
constexpr int kRowWideCols = 8192;
static_assert(kRowMaxRegisterCols <= 8 * 4 * 1024, "wide rows: at most 8 float4 per thread");

// Launchers return hipSuccess or the launch error.
hipError_t launch_cast(const CastArgs& a, hipStream_t s);
hipError_t launch_frob(const FrobArgs& a, hipStream_t s);
enum GemmTile : int { kTileSmall = 0, kTileBig = 1 };
hipError_t launch_ns_gemm(GemmMode mode, GemmTile tile, const NsArgs& a, hipStream_t s);
hipError_t launch_rownorm_rows(const RowArgs& a, int max_cols, bool vec, hipStream_t s);
hipError_t launch_rownorm_rows_wide(const RowArgs& a, int max_cols, hipStream_t s);
hipError_t launch_colnorm_partial(const ColArgs& a, bool vec, hipStream_t s);
hipError_t launch_colnorm_finalize(const ColArgs& a, int fin_total, hipStream_t s);
hipError_t launch_colnorm_apply(const ColArgs& a, bool vec, hipStream_t s);
hipError_t launch_rms_finalize(const RmsArgs& a, hipStream_t s);
hipError_t launch_adamw(const AdamArgs& a, hipStream_t s);
hipError_t launch_scaled_update(const UpdArgs& a, hipStream_t s);
hipError_t launch_sp_gram(const SpArgs& a, hipStream_t s);
hipError_t launch_sp_house(const SpArgs& a, hipStream_t s);
hipError_t launch_sp_pass(const SpArgs& a, int max_tiles, hipStream_t s);
hipError_t launch_sp_reduce(const SpArgs& a, int max_trailing, hipStream_t s);
hipError_t launch_sp_bisect(const SpArgs& a, int max_m, hipStream_t s);
hipError_t launch_sp_entropy(const SpArgs& a, hipStream_t s);

// GEMM block tiles (host-side tile counting must match the kernels).
#ifndef MUON_GEMM_BIG_M
#define MUON_GEMM_BIG_M 256
#endif
#ifndef MUON_GEMM_BIG_N
#define MUON_GEMM_BIG_N 256
#endif
constexpr int kGemmSmall = 128;
constexpr int kGemmBigM = MUON_GEMM_BIG_M;
constexpr int kGemmBigN = MUON_GEMM_BIG_N;
// A stage uses the big tile when it has at least this many big tiles.
#ifndef MUON_GEMM_BIG_MIN_TILES
#define MUON_GEMM_BIG_MIN_TILES 512
#endif
constexpr int kGemmBigMinTiles = MUON_GEMM_BIG_MIN_TILES;
// The Gram takes the big tile from this many big tiles on: on big tiles it reads X_c
// (transposing LDS reads), so the cast and the Apply then skip the row-major X copy.
#ifndef MUON_GEMM_BIG_MIN_TILES_GRAM
#define MUON_GEMM_BIG_MIN_TILES_GRAM 128
#endif
constexpr int kGemmBigMinTilesGram = MUON_GEMM_BIG_MIN_TILES_GRAM;

}  // namespace muon
