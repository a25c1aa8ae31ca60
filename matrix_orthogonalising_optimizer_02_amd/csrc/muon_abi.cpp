// C ABI of libmuon_rocm: argument validation, bucket planning, workspace layout,
// kernel dispatch and optional per-kernel timing. Declared in include/muon_rocm.h.
//
// Step structure (Muon notes Sec. 2.1 Eq. 1-2, Sec. 2.2 Eq. 4; DiT paper, Periodic
// Row-wise paragraphs):
//   refresh step:  cast (M <- mu M + G, ||M||^2 partials, bf16 X_r / X_c)
//                  -> frob (s = 1 / max(||M||_F, eps))
//                  -> N x [gram, poly, apply]; the last apply applies Eq. 4 (Eq. 5) to W,
//                     or, under Eq. 6 (Sec. 3.1), writes fp32 O over the two X_r buffers
//                     (free by then) -> RMS(O) -> W <- decay W - lr 0.2 / RMS(O) O
//   RowNorm step:  rows kernel (flat / square) or partial -> finalize -> apply (tall)
//   update-RMS monitor (optional): the last apply / the RowNorm kernels leave partial
//                  sums of U^2 in the workspace; one finalize kernel per group reduces them
// Matrices are planned in groups of up to kMaxGroup, ordered by working size m and
// then by n (largest first), and each group's kernels cover all of its matrices in
// one launch per stage. Groups run one after another on the caller's stream and
// reuse the same workspace region.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon_rocm.h"
#include "abi_internal.hpp"
#include "launch.hpp"

#define MUON_API extern "C" __attribute__((visibility("default")))

namespace muon {
namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& what) {
    g_last_error = what;
    return code;
}

constexpr int64_t kMaxDim = int64_t(1) << 30;
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int kMaxNsSteps = 100;

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- planning ----
struct MatPlan {
    int idx;                  // caller's index
    int64_t rows, cols;
    bool tall;                // rows > cols
    int64_t m, n, m_p, n_p;   // working dims and padded dims
    int64_t rows_p, cols_p;   // padded dims in the input orientation
    int64_t cast_tiles;
    int64_t max_tiles;        // final-apply tiles with the smallest tile (partial sums)
    // workspace offsets (relative to the group base)
    size_t xr[2], xc[2], a, b, partial, scale;  // refresh; xr[0], xr[1] are adjacent
    size_t rpart, coef;                         // refresh: per-wave O^2 sums, Eq. 6 factor
    size_t colpart, inv;                        // RowNorm, tall only
    size_t rpart_rn;                            // RowNorm: per-line R^2 sums
    int64_t chunks;
};

struct GroupPlan {
    std::vector<MatPlan> mats;
    size_t bytes = 0;
    size_t rn_bytes = 0;      // the part the RowNorm step uses (column partials, norms, monitor)
    size_t tail = 0;          // fp32 partial tiles of the stages that split their tail
    int64_t tail_units = 0;
};

// MI355X: 256 compute units in 8 XCDs; a big-tile block fills one compute unit.
constexpr int kCusPerXcd = 32;

// Tail split of a GEMM stage on big tiles. XCD x runs cnt[x] tiles in rounds of
// kCusPerXcd blocks; a last round of r <= kCusPerXcd / 2 tiles would leave most of the
// XCD idle while it runs, so those r tiles run as S chunks of K each (S r <= kCusPerXcd,
// S <= kTailMaxSplit, chunks cut at multiples of 256 of K, i.e. of 8 K steps). The split
// is taken only when the time it saves, (1 - 1 / S) of a tile for the XCD that splits
// least, exceeds what its partial tiles cost (one fp32 tile written and read per chunk,
// plus the fixup launch); the constants are measured on MI355X. Returns the number of
// partial tiles (0: no split).
constexpr double kTailStepUs = 0.86;   // one 32-wide K step of a 256 x 256 tile
constexpr double kTailUnitUs = 0.13;   // 512 KiB of partial-tile traffic
constexpr double kTailFixedUs = 10.0;  // the fixup launch
int64_t tail_split(const int64_t cnt[8], int64_t ksteps, NsArgs* na) {
    int64_t S[8], tail[8], units = 0, s_min = kTailMaxSplit;
    for (int x = 0; x < 8; ++x) {
        const int64_t r = cnt[x] % kCusPerXcd;
        S[x] = 1;
        if (r > 0 && r <= kCusPerXcd / 2)
            S[x] = std::min<int64_t>({kTailMaxSplit, kCusPerXcd / r, ksteps / 8});
        if (S[x] < 2) S[x] = 1;
        tail[x] = S[x] > 1 ? r : 0;
        if (tail[x]) s_min = std::min(s_min, S[x]);
        units += tail[x] * S[x];
    }
    const double saved = (1.0 - 1.0 / double(s_min)) * double(ksteps) * kTailStepUs;
    if (units == 0 || saved <= double(units) * kTailUnitUs + kTailFixedUs) {
        units = 0;
        for (int x = 0; x < 8; ++x) { S[x] = 1; tail[x] = 0; }
    }
    if (na) {
        int64_t base = 0;
        for (int x = 0; x < 8; ++x) {
            na->xfull[x] = int32_t(cnt[x] - tail[x]);
            na->xtail[x] = int32_t(tail[x]);
            na->xsplit[x] = int32_t(S[x]);
            na->xpbase[x] = int32_t(base);
            base += tail[x] * S[x];
        }
    }
    return units;
}

enum SplitStage : int { kStageGram = 0, kStagePoly = 1, kStageApply = 2 };

// Tiles of eighth j of a sequence of T tiles.
inline int64_t eighth(int64_t T, int64_t j) { return ((j + 1) * T >> 3) - (j * T >> 3); }

// Tiles of matrix p in a stage on `tile`-wide tiles (upper-triangle tiles for the Gram
// and polynomial, all tiles of X' for the Apply) and their K in units of 256 (Gram: n_p;
// polynomial and Apply: m_p).
int64_t stage_tiles(const MatPlan& p, int stage, int64_t tile) {
    const int64_t t = p.m_p / tile;
    return stage == kStageApply ? t * (p.n_p / tile) : t * (t + 1) / 2;
}
int64_t stage_k(const MatPlan& p, int stage) { return (stage == kStageGram ? p.n_p : p.m_p) / 256; }

// How a stage's tiles are dealt to the 8 XCDs. Each XCD takes one contiguous eighth of
// every matrix's tile sequence, so neighbouring tiles, which share operand panels, meet
// in its L2: eighth (x + rot) & 7 goes to XCD x. Eighths of a sequence whose length is
// not a multiple of 8 differ by one tile. The balanced deal gives each matrix, in group
// order, the rotation that leaves the XCDs' loads (tiles x K) with the smallest sum of
// squares, the first one on a tie; the plain deal rotates nothing, so the same XCDs
// take the larger eighth of every matrix (the 16-matrix [2048, 8192] bucket's Gram: 80
// tiles on four XCDs, 64 on the others).
struct XcdDeal {
    int32_t rot[kMaxGroup];
    int64_t cnt[8];
};
XcdDeal xcd_deal(const GroupPlan& gp, int stage, int64_t tile, bool balance) {
    XcdDeal d{};
    int64_t load[8] = {0};
    for (size_t g = 0; g < gp.mats.size(); ++g) {
        const int64_t T = stage_tiles(gp.mats[g], stage, tile), k = stage_k(gp.mats[g], stage);
        int best_r = 0;
        int64_t best = -1;
        for (int r = 0; balance && r < 8; ++r) {
            int64_t v = 0;
            for (int x = 0; x < 8; ++x) {
                const int64_t l = load[x] + eighth(T, (x + r) & 7) * k;
                v += l * l;
            }
            if (best < 0 || v < best) {
                best = v;
                best_r = r;
            }
        }
        d.rot[g] = best_r;
        for (int x = 0; x < 8; ++x) {
            const int64_t e = eighth(T, (x + best_r) & 7);
            d.cnt[x] += e;
            load[x] += e * k;
        }
    }
    return d;
}

// Per XCD, the K (units of 256) of each big tile it takes, in order.
void xcd_seqs(const GroupPlan& gp, int stage, const XcdDeal& deal, std::vector<int64_t> ks[8]) {
    for (int x = 0; x < 8; ++x) ks[x].clear();
    for (size_t g = 0; g < gp.mats.size(); ++g) {
        const int64_t T = stage_tiles(gp.mats[g], stage, kGemmBigM), k = stage_k(gp.mats[g], stage);
        for (int x = 0; x < 8; ++x) ks[x].insert(ks[x].end(), size_t(eighth(T, (x + deal.rot[g]) & 7)), k);
    }
}

// The stage's K in 32-wide steps when every matrix of the group has the same K, else 0.
int64_t shared_ksteps(const GroupPlan& gp, int stage) {
    int64_t k = -1;
    for (const MatPlan& p : gp.mats) {
        const int64_t kp = stage_k(p, stage);
        if (k < 0) k = kp;
        else if (k != kp) k = 0;
    }
    return k > 0 ? k * 8 : 0;
}

// Head split of a stage on big tiles whose matrices have different K and whose tiles all
// fit one round (at most kCusPerXcd per XCD): the XCD's tiles all start together, so the
// stage lasts as long as its longest tile, the first ones of its sequence (the group runs
// longest K first). XCD x runs its first h tiles as S chunks of K each (blocks 0 .. h S - 1,
// its other tiles after them), within one round: h S + cnt - h <= kCusPerXcd, and every
// split tile at least S units of 256 of K long. Its longest block is then max(ceil(k_i / S)
// over the split tiles, k_i over the others), k in units of 256. The stage's target is the
// largest over the XCDs of the smallest such value; each XCD then takes, among the (h, S)
// that reach the target, the one with the fewest partial tiles (then the fewest chunks).
// Taken, like the tail split, when the K steps saved on the longest XCD beat the
// partial-tile cost. Measured on the H = 2048 DiT block's Gram (the odd XCDs' 25 tiles of
// 48 to 8 units: 48 -> 32). Returns the number of partial tiles (0: no split); *span
// (optional) receives the longest block in units of 256 of K.
int64_t head_split(const std::vector<int64_t> ks[8], NsArgs* na, int64_t* span = nullptr) {
    // per XCD: the longest block of a split of the first h tiles into S chunks
    auto longest = [&](const std::vector<int64_t>& v, int64_t h, int64_t S) {
        int64_t l = 0;
        for (int64_t i = 0; i < int64_t(v.size()); ++i)
            l = std::max(l, i < h ? (v[size_t(i)] + S - 1) / S : v[size_t(i)]);
        return l;
    };
    auto fits = [&](const std::vector<int64_t>& v, int64_t h, int64_t S) {
        if (h * S + int64_t(v.size()) - h > kCusPerXcd) return false;
        for (int64_t i = 0; i < h; ++i)
            if (v[size_t(i)] < S) return false;
        return true;
    };
    int64_t before = 0, target = 0;
    for (int x = 0; x < 8; ++x) {
        if (int64_t(ks[x].size()) > kCusPerXcd) return 0;
        const int64_t l0 = longest(ks[x], 0, 1);
        int64_t best = l0;
        for (int64_t S = 2; S <= kTailMaxSplit; ++S)
            for (int64_t h = 1; h <= int64_t(ks[x].size()) && fits(ks[x], h, S); ++h)
                best = std::min(best, longest(ks[x], h, S));
        before = std::max(before, l0);
        target = std::max(target, best);
    }
    if (span) *span = before;
    int64_t H[8], SS[8], units = 0;
    for (int x = 0; x < 8; ++x) {
        H[x] = 0;
        SS[x] = 1;
        if (longest(ks[x], 0, 1) <= target) continue;
        for (int64_t S = 2; S <= kTailMaxSplit; ++S)
            for (int64_t h = 1; h <= int64_t(ks[x].size()) && fits(ks[x], h, S); ++h)
                if (longest(ks[x], h, S) <= target && (H[x] == 0 || h * S < H[x] * SS[x])) {
                    H[x] = h;
                    SS[x] = S;
                }
        units += H[x] * SS[x];
    }
    const double saved = double((before - target) * 8) * kTailStepUs;
    if (units == 0 || saved <= double(units) * kTailUnitUs + kTailFixedUs) return 0;
    if (span) *span = target;
    if (na) {
        int64_t base = 0;
        for (int x = 0; x < 8; ++x) {
            na->xfull[x] = 0;
            na->xtail[x] = int32_t(H[x]);
            na->xsplit[x] = int32_t(SS[x]);
            na->xpbase[x] = int32_t(base);
            base += H[x] * SS[x];
        }
    }
    return units;
}

// Modelled time of a stage on big tiles under a deal, in hundredths of a microsecond:
// the busiest XCD's span in K steps at kTailStepUs each, plus the partial-tile cost of
// the split the planner takes under that deal. An XCD runs its blocks on kCusPerXcd
// compute units, each block on the first one free, in order: with one K the span is
// q K plus the last round's (chunked) tiles; with mixed K and one round it is the
// longest block; with mixed K and more rounds it is found by that list schedule.
int64_t deal_cost(const GroupPlan& gp, int stage, const XcdDeal& deal) {
    constexpr int64_t kStep = 86, kUnit = 13, kFixed = 1000;  // kTailStepUs, kTailUnitUs, kTailFixedUs
    const int64_t ksteps = shared_ksteps(gp, stage);
    int64_t span = 0, units = 0;
    if (ksteps) {
        NsArgs na{};
        int64_t cnt[8];
        for (int x = 0; x < 8; ++x) cnt[x] = deal.cnt[x];
        units = tail_split(cnt, ksteps, &na);
        for (int x = 0; x < 8; ++x) {
            const int64_t q = cnt[x] / kCusPerXcd, r = cnt[x] % kCusPerXcd;
            const int64_t last = (units > 0 && na.xtail[x] > 0) ? (ksteps / 8 + na.xsplit[x] - 1) / na.xsplit[x] * 8
                                                                : (r > 0 ? ksteps : 0);
            span = std::max(span, q * ksteps + last);
        }
    } else {
        std::vector<int64_t> ks[8];
        xcd_seqs(gp, stage, deal, ks);
        int64_t longest = 0;
        units = head_split(ks, nullptr, &longest);
        if (longest > 0) {
            span = longest * 8;
        } else {
            for (int x = 0; x < 8; ++x) {
                int64_t free_at[kCusPerXcd] = {0};
                for (const int64_t k : ks[x]) {
                    int64_t* cu = std::min_element(free_at, free_at + kCusPerXcd);
                    *cu += k * 8;
                    span = std::max(span, *cu);
                }
            }
        }
    }
    return span * kStep + (units > 0 ? units * kUnit + kFixed : 0);
}

// The deal of a stage: on small tiles (no split) the balanced one; on big tiles the
// balanced one when its modelled time is below the plain deal's. Balancing alone can
// lose: 16 [2048, 2048] matrices go from 64 or 80 tiles per XCD (the 80 split in two
// chunks) to 72 everywhere, whose last round of 8 short tiles does not pay for a split.
XcdDeal stage_deal(const GroupPlan& gp, int stage, int64_t tile) {
    const XcdDeal bal = xcd_deal(gp, stage, tile, true);
    if (tile != kGemmBigM) return bal;
    bool rotated = false;
    for (size_t g = 0; g < gp.mats.size(); ++g) rotated = rotated || bal.rot[g] != 0;
    if (!rotated) return bal;
    const XcdDeal plain = xcd_deal(gp, stage, tile, false);
    return deal_cost(gp, stage, bal) < deal_cost(gp, stage, plain) ? bal : plain;
}

// The split of a stage on big tiles under its deal: the tail split when its matrices
// share K, else the head split (with mixed K the last tiles of an XCD are its shortest
// ones and splitting them was measured to cost more than it saves). *head (optional)
// tells which.
int64_t split_plan(const GroupPlan& gp, int stage, NsArgs* na, bool* head = nullptr) {
    const XcdDeal deal = stage_deal(gp, stage, kGemmBigM);
    const int64_t ksteps = shared_ksteps(gp, stage);
    if (head) *head = ksteps == 0;
    if (ksteps) {
        int64_t cnt[8];
        for (int x = 0; x < 8; ++x) cnt[x] = deal.cnt[x];
        return tail_split(cnt, ksteps, na);
    }
    std::vector<int64_t> ks[8];
    xcd_seqs(gp, stage, deal, ks);
    return head_split(ks, na);
}

// Big tiles of a stage, the first test of choose_tile.
int64_t big_tiles(const GroupPlan& gp, bool sym) {
    int64_t big = 0;
    for (const MatPlan& p : gp.mats) {
        const int64_t t = p.m_p / kGemmBigM;
        big += sym ? t * (t + 1) / 2 : t * (p.n_p / kGemmBigN);
    }
    return big;
}

// The tile of a GEMM stage: big (256 x 256, one block per compute unit) when the stage
// has at least kGemmBigMinTiles of them (kGemmBigMinTilesGram for the Gram, whose big
// tiles also spare the cast and the Apply the row-major X copy: the H = 2048 DiT block's
// Gram, 180 big tiles of mixed K, moved to big tiles took its vanilla step 3.19 -> 3.03
// ms, Apply +11%); also when its tiles all have the same K (the
// polynomial and the Apply, whose K is m, when every matrix of the group has the same
// m; the Gram when they have the same n) and the big tiles need fewer rounds on the
// busiest XCD than the small ones (128 x 128, two blocks per compute unit); small
// otherwise. Measured: ns5_batched on [4096, 4096] 1.79 -> 1.51 ms (Gram, polynomial
// and Apply each one round of big tiles against two of small ones); one [6144, 6144]
// 5.20 -> 4.27 ms and two [4096, 4096] 3.34 -> 2.67 ms (the Gram and polynomial two
// rounds against three, their short last round then split); the H = 2048 block's
// polynomial 0.080 -> 0.068 ms per launch. Both tiles accumulate over K in the same order with the same
// epilogue arithmetic, so the choice alone changes no result.
GemmTile choose_tile(const GroupPlan& gp, bool sym, int stage) {
    const int ng = int(gp.mats.size());
    const bool big_ok = !sym || kGemmBigM == kGemmBigN;
    if (!big_ok || ng == 0) return kTileSmall;
    if (big_tiles(gp, sym) >= ((sym && stage == kStageGram) ? kGemmBigMinTilesGram : kGemmBigMinTiles)) return kTileBig;
    bool same_m = true, same_n = true;
    for (int k = 1; k < ng; ++k) {
        same_m = same_m && gp.mats[k].m_p == gp.mats[0].m_p;
        same_n = same_n && gp.mats[k].n_p == gp.mats[0].n_p;
    }
    if (!((sym && stage == kStageGram) ? same_n : same_m)) return kTileSmall;
    const int st = sym ? stage : int(kStageApply);
    const XcdDeal db = stage_deal(gp, st, kGemmBigM), ds = stage_deal(gp, st, kGemmSmall);
    const int64_t mb = *std::max_element(db.cnt, db.cnt + 8), ms = *std::max_element(ds.cnt, ds.cnt + 8);
    const int64_t rounds_big = (mb + kCusPerXcd - 1) / kCusPerXcd;
    const int64_t rounds_small = (ms + 2 * kCusPerXcd - 1) / (2 * kCusPerXcd);
    return (mb > 0 && rounds_big < rounds_small) ? kTileBig : kTileSmall;
}

struct Plan {
    std::vector<GroupPlan> groups;
    size_t bytes = 0;
    size_t rn_bytes = 0;      // the largest group's RowNorm part
};

int make_plan(const int64_t* rows, const int64_t* cols, int32_t count, Plan* plan) {
    std::vector<MatPlan> all;
    for (int i = 0; i < count; ++i) {
        const int64_t r = rows[i], c = cols[i];
        if (r < 0 || c < 0) return fail(MUON_ERR_INVALID_ARG, "negative matrix dimension at index " + std::to_string(i));
        if (r == 0 || c == 0) continue;
        if (r > kMaxDim || c > kMaxDim || r * c > kMaxElems)
            return fail(MUON_ERR_TOO_LARGE, "matrix " + std::to_string(i) + " exceeds the size limits");
        MatPlan p{};
        p.idx = i;
        p.rows = r;
        p.cols = c;
        p.tall = r > c;
        p.m = std::min(r, c);
        p.n = std::max(r, c);
        p.m_p = round_up(p.m, kPad);
        p.n_p = round_up(p.n, kPad);
        p.rows_p = p.tall ? p.n_p : p.m_p;
        p.cols_p = p.tall ? p.m_p : p.n_p;
        p.cast_tiles = (p.rows_p / 64) * (p.cols_p / 64);
        p.max_tiles = (p.m_p / kGemmSmall) * (p.n_p / kGemmSmall);
        p.chunks = (r + kColChunkRows - 1) / kColChunkRows;
        all.push_back(p);
    }
    std::stable_sort(all.begin(), all.end(), [](const MatPlan& x, const MatPlan& y) {
        if (x.m != y.m) return x.m > y.m;
        return x.n > y.n;
    });
    plan->groups.clear();
    plan->bytes = 0;
    plan->rn_bytes = 0;
    for (size_t s = 0; s < all.size(); s += kMaxGroup) {
        GroupPlan gp;
        size_t ns = 0, rn = 0;
        int64_t cast_total = 0, rows_total = 0, col_total = 0, upd_total = 0;
        for (size_t k = s; k < std::min(all.size(), s + kMaxGroup); ++k) {
            MatPlan p = all[k];
            const size_t xbytes = size_t(p.m_p) * size_t(p.n_p) * 2;
            const size_t abytes = size_t(p.m_p) * size_t(p.m_p) * 2;
            // xbytes is a multiple of 256: xr[1] starts where xr[0] ends, so together they
            // hold an fp32 [rows, cols] O for the Eq. 6 update
            for (int q = 0; q < 2; ++q) { p.xr[q] = ns; ns = align256(ns + xbytes); }
            for (int q = 0; q < 2; ++q) { p.xc[q] = ns; ns = align256(ns + xbytes); }
            p.a = ns; ns = align256(ns + abytes);
            p.b = ns; ns = align256(ns + abytes);
            p.partial = ns; ns = align256(ns + size_t(p.cast_tiles) * 4);
            p.scale = ns; ns = align256(ns + 4);
            p.rpart = ns; ns = align256(ns + size_t(p.max_tiles) * 4 * 4);
            p.coef = ns; ns = align256(ns + 4);
            p.rpart_rn = rn; rn = align256(rn + size_t(p.tall ? p.cols : p.rows) * 4);
            if (p.tall) {
                p.colpart = rn; rn = align256(rn + size_t(p.chunks) * size_t(p.cols) * 4);
                p.inv = rn; rn = align256(rn + size_t(p.cols) * 4);
                col_total += p.chunks * ((p.cols + kColTileCols - 1) / kColTileCols);
            } else {
                rows_total += p.rows;
            }
            cast_total += p.cast_tiles;
            upd_total += (p.rows * p.cols + kUpdBlockElems - 1) / kUpdBlockElems;
            gp.mats.push_back(p);
        }
        const int64_t tile_total_cap = int64_t(1) << 31;
        if (cast_total >= tile_total_cap || rows_total >= tile_total_cap || col_total >= tile_total_cap ||
            upd_total >= tile_total_cap)
            return fail(MUON_ERR_TOO_LARGE, "a launch would exceed 2^31 workgroups");
        if (kGemmTailSplit) {
            // the partial-tile region serves whichever stage splits the most tiles
            gp.tail_units = 0;
            for (int st = kStageGram; st <= kStageApply; ++st) {
                if (choose_tile(gp, st != kStageApply, st) != kTileBig) continue;
                gp.tail_units = std::max(gp.tail_units, split_plan(gp, st, nullptr));
            }
            if (gp.tail_units > 0) {
                gp.tail = ns;
                ns = align256(ns + size_t(gp.tail_units) * kTailUnitFloats * 4);
            }
        }
        gp.bytes = std::max(ns, rn);
        gp.rn_bytes = rn;
        plan->bytes = std::max(plan->bytes, gp.bytes);
        plan->rn_bytes = std::max(plan->rn_bytes, rn);
        plan->groups.push_back(std::move(gp));
    }
    return MUON_OK;
}

// ---------------------------------------------------------------- timing ----
struct TimingRecord {
    int cls;
    hipEvent_t start, stop;
};

struct Timing {
    std::mutex mu;
    bool enabled = false;
    std::vector<TimingRecord> records;
    std::vector<hipEvent_t> pool;
} g_timing;

// Nonzero while a call that must not create events (the allocation-free entry point)
// enqueues its kernels: the timing facility then leaves them unbracketed.
thread_local int g_untimed = 0;

hipEvent_t take_event() {
    if (!g_timing.pool.empty()) {
        hipEvent_t e = g_timing.pool.back();
        g_timing.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

template <class F>
int run_kernel(int cls, hipStream_t s, const char* name, F&& launch) {
    hipEvent_t a = nullptr, b = nullptr;
    bool timed = false;
    {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        if (g_timing.enabled && !g_untimed) {
            a = take_event();
            b = take_event();
            timed = a && b;
            if (timed && hipEventRecord(a, s) != hipSuccess) timed = false;
        }
    }
    const hipError_t e = launch();
    if (e != hipSuccess) return fail(MUON_ERR_HIP, std::string(name) + ": " + hipGetErrorString(e));
    if (timed) {
        std::lock_guard<std::mutex> lk(g_timing.mu);
        if (hipEventRecord(b, s) == hipSuccess) g_timing.records.push_back({cls, a, b});
    }
    return MUON_OK;
}

// ---------------------------------------------------------------- checks ----
int check_hparams(const muon_hparams* hp, bool need_steps) {
    if (!hp) return fail(MUON_ERR_INVALID_ARG, "hparams is NULL");
    if (!(hp->eps > 0.f) || !std::isfinite(hp->eps)) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (hp->ns_steps < 1 || hp->ns_steps > kMaxNsSteps)
        return fail(MUON_ERR_INVALID_ARG, "ns_steps must be in [1, 100]");
    if (need_steps && hp->period_k < 1) return fail(MUON_ERR_INVALID_ARG, "period_k must be >= 1");
    if (hp->scale_mode != MUON_SCALE_MAX_DIM && hp->scale_mode != MUON_SCALE_HIDDEN &&
        hp->scale_mode != MUON_SCALE_RMS)
        return fail(MUON_ERR_INVALID_ARG, "unknown scale_mode");
    if (hp->scale_mode == MUON_SCALE_HIDDEN && hp->hidden < 1)
        return fail(MUON_ERR_INVALID_ARG, "hidden must be >= 1 under MUON_SCALE_HIDDEN");
    return MUON_OK;
}

// The factor of the update direction before the learning rate (Eq. 4 / Eq. 5; the
// Eq. 6 refresh factor is computed on the device).
double dir_scale(const muon_hparams& hp, int64_t n) {
    const double h = hp.scale_mode == MUON_SCALE_HIDDEN ? double(hp.hidden) : double(n);
    return double(hp.rms_scale) * std::sqrt(h);
}

struct Range {
    uintptr_t lo, hi;
    bool write;
};

int check_overlaps(std::vector<Range>& rs) {
    std::sort(rs.begin(), rs.end(), [](const Range& x, const Range& y) { return x.lo < y.lo; });
    uintptr_t hi_any = 0, hi_write = 0;
    for (const Range& r : rs) {
        if (r.hi <= r.lo) continue;
        if (r.lo < (r.write ? hi_any : hi_write)) return fail(MUON_ERR_ALIAS, "buffers overlap");
        hi_any = std::max(hi_any, r.hi);
        if (r.write) hi_write = std::max(hi_write, r.hi);
    }
    return MUON_OK;
}

int check_monitor(const float* update_rms, int32_t count, std::vector<Range>& ranges) {
    if (!update_rms || count == 0) return MUON_OK;
    if (reinterpret_cast<uintptr_t>(update_rms) & 3) return fail(MUON_ERR_ALIGN, "update_rms not 4-byte aligned");
    const uintptr_t lo = reinterpret_cast<uintptr_t>(update_rms);
    ranges.push_back({lo, lo + uintptr_t(count) * 4, true});
    return MUON_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int check_workspace(const Plan& plan, void* ws, size_t ws_bytes, std::vector<Range>& ranges) {
    if (plan.bytes == 0) return MUON_OK;
    if (!ws) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if (ws_bytes < plan.bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(plan.bytes) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MUON_ERR_ALIGN, "workspace not 256-byte aligned");
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ws);
    ranges.push_back({lo, lo + plan.bytes, true});
    return MUON_OK;
}

int check_matrices(const muon_matrix* mats, int32_t count, std::vector<int64_t>& rows,
                   std::vector<int64_t>& cols, std::vector<Range>& ranges) {
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && !mats) return fail(MUON_ERR_INVALID_ARG, "mats is NULL");
    rows.resize(count);
    cols.resize(count);
    for (int i = 0; i < count; ++i) {
        const muon_matrix& t = mats[i];
        rows[i] = t.rows;
        cols[i] = t.cols;
        if (t.rows < 0 || t.cols < 0) return fail(MUON_ERR_INVALID_ARG, "negative dimension at index " + std::to_string(i));
        if (t.rows == 0 || t.cols == 0) continue;
        if (t.rows > kMaxDim || t.cols > kMaxDim || t.rows * t.cols > kMaxElems)
            return fail(MUON_ERR_TOO_LARGE, "matrix " + std::to_string(i) + " exceeds the size limits");
        if (!t.w || !t.m || !t.g) return fail(MUON_ERR_INVALID_ARG, "NULL w, m or g at index " + std::to_string(i));
        if (!aligned16(t.w) || !aligned16(t.m) || !aligned16(t.g))
            return fail(MUON_ERR_ALIGN, "matrix pointer not 16-byte aligned at index " + std::to_string(i));
        const uintptr_t bytes = uintptr_t(t.rows) * uintptr_t(t.cols) * 4;
        ranges.push_back({reinterpret_cast<uintptr_t>(t.w), reinterpret_cast<uintptr_t>(t.w) + bytes, true});
        ranges.push_back({reinterpret_cast<uintptr_t>(t.m), reinterpret_cast<uintptr_t>(t.m) + bytes, true});
        ranges.push_back({reinterpret_cast<uintptr_t>(t.g), reinterpret_cast<uintptr_t>(t.g) + bytes, false});
    }
    return MUON_OK;
}

// ---------------------------------------------------------------- dispatch ----
struct IoPtrs {
    const float* m_in;
    const float* g;
    float* m_out;
    float* out;  // W (fused update) or O
};

// Fills tiles / tile_begin / total of a GEMM stage launch and returns the tile
// configuration that choose_tile picks for the stage.
// ws != nullptr: the stage (Gram, polynomial or a non-final Apply) may split its tail
// tiles into the workspace's partial-tile region. describe: plan that split without a
// workspace (ns5_plan reads xtail / xsplit; na.tail stays NULL).
GemmTile plan_tiles(const GroupPlan& gp, NsArgs& na, bool sym, char* ws = nullptr, int stage = kStageGram,
                    bool describe = false, bool* head = nullptr) {
    const int ng = int(gp.mats.size());
    const GemmTile tile = choose_tile(gp, sym, stage);
    const int64_t bm = tile == kTileBig ? kGemmBigM : kGemmSmall;
    const int64_t bn = tile == kTileBig ? kGemmBigN : kGemmSmall;
    for (int k = 0; k < ng; ++k) {
        const MatPlan& p = gp.mats[k];
        if (sym) {
            const int64_t t = p.m_p / bm;
            na.d[k].tiles = int32_t(t);
            na.d[k].ntiles = int32_t(t * (t + 1) / 2);
        } else {
            na.d[k].tiles = int32_t(p.n_p / bn);
            na.d[k].ntiles = int32_t((p.m_p / bm) * (p.n_p / bn));
        }
    }
    // the kernels deal each matrix's tiles over the 8 XCDs in rotated contiguous eighths
    const XcdDeal deal = stage_deal(gp, sym ? stage : int(kStageApply), bm);
    int64_t per_xcd_max = 0;
    for (int k = 0; k < ng; ++k) na.d[k].rot = deal.rot[k];
    for (int x = 0; x < 8; ++x) per_xcd_max = std::max(per_xcd_max, deal.cnt[x]);
    const int64_t tot = 8 * per_xcd_max;
    na.total = int32_t(tot);
    na.tail = nullptr;
    na.fix_total = 0;
    if (tile == kTileBig && (ws != nullptr || describe) && gp.tail_units > 0) {
        int64_t fix = 0, longest = 0;
        const int64_t units = split_plan(gp, stage, &na, head);
        if (units > 0 && units <= gp.tail_units) {
            for (int x = 0; x < 8; ++x) {
                fix += na.xtail[x];
                longest = std::max<int64_t>(longest, deal.cnt[x] + int64_t(na.xtail[x]) * (na.xsplit[x] - 1));
            }
            na.tail = ws ? reinterpret_cast<float*>(ws + gp.tail) : nullptr;
            na.fix_total = int32_t(fix);
            na.total = int32_t(8 * longest);
        }
    }
    return tile;
}

// Copies a planned stage's tiling (tile counts, XCD rotations, grid, split) into the
// launch arguments.
void take_tiling(NsArgs& na, const NsArgs& plan, int ng) {
    for (int k = 0; k < ng; ++k) {
        na.d[k].tiles = plan.d[k].tiles;
        na.d[k].ntiles = plan.d[k].ntiles;
        na.d[k].rot = plan.d[k].rot;
    }
    na.total = plan.total;
    na.tail = plan.tail;
    na.fix_total = plan.fix_total;
    std::memcpy(na.xfull, plan.xfull, sizeof(na.xfull));
    std::memcpy(na.xtail, plan.xtail, sizeof(na.xtail));
    std::memcpy(na.xsplit, plan.xsplit, sizeof(na.xsplit));
    std::memcpy(na.xpbase, plan.xpbase, sizeof(na.xpbase));
}

int run_refresh(const GroupPlan& gp, const std::vector<IoPtrs>& io, const muon_hparams& hp,
                bool momentum, bool update_w, char* ws, float* update_rms, hipStream_t s) {
    const int ng = int(gp.mats.size());
    const bool eq6 = update_w && hp.scale_mode == MUON_SCALE_RMS;
    const bool monitor = update_w && update_rms != nullptr;
    // The big-tile Gram reads X_c (transposing LDS reads), so X_r, the row-major copy, is
    // produced only when this group's Gram runs on small tiles.
    NsArgs probe{};
    const bool need_xr = plan_tiles(gp, probe, true) == kTileSmall;
    // cast
    CastArgs ca{};
    ca.n = ng;
    ca.mu = hp.mu;
    ca.use_momentum = momentum ? 1 : 0;
    int64_t tiles = 0;
    for (int k = 0; k < ng; ++k) {
        const MatPlan& p = gp.mats[k];
        CastDesc& d = ca.d[k];
        d.m_in = io[k].m_in;
        d.g = io[k].g;
        d.m_out = io[k].m_out;
        unsigned short* xr = reinterpret_cast<unsigned short*>(ws + p.xr[0]);
        unsigned short* xc = reinterpret_cast<unsigned short*>(ws + p.xc[0]);
        d.direct = p.tall ? xc : (need_xr ? xr : nullptr);
        d.transp = p.tall ? (need_xr ? xr : nullptr) : xc;
        d.direct_blk = p.tall ? 1 : 0;  // X_c is panel-blocked, X_r row-major
        d.transp_blk = p.tall ? 0 : 1;
        d.partial = reinterpret_cast<float*>(ws + p.partial);
        d.rows = int32_t(p.rows);
        d.cols = int32_t(p.cols);
        d.rows_p = int32_t(p.rows_p);
        d.cols_p = int32_t(p.cols_p);
        d.tiles_c = int32_t(p.cols_p / 64);
        d.wide = d.transp == nullptr ? 1 : 0;  // cols_p is a multiple of 256
        d.tile_begin = int32_t(tiles);
        tiles += p.cast_tiles;
    }
    ca.total = int32_t(tiles);
    int rc = run_kernel(MUON_KCLASS_CAST, s, "cast", [&] { return launch_cast(ca, s); });
    if (rc) return rc;

    FrobArgs fa{};
    fa.n = ng;
    fa.eps = hp.eps;
    for (int k = 0; k < ng; ++k) {
        const MatPlan& p = gp.mats[k];
        fa.partial[k] = reinterpret_cast<const float*>(ws + p.partial);
        fa.scale[k] = reinterpret_cast<float*>(ws + p.scale);
        fa.count[k] = int32_t(p.cast_tiles);
    }
    rc = run_kernel(MUON_KCLASS_FROB, s, "frob", [&] { return launch_frob(fa, s); });
    if (rc) return rc;

    NsArgs na{};
    na.n = ng;
    na.ca = hp.ns_a;
    na.cb = hp.ns_b;
    na.cc = hp.ns_c;
    na.decay = 1.0f - hp.lr * hp.weight_decay;
    // the stages' tilings, the same in every iteration
    NsArgs plan_gram{}, plan_poly{}, plan_apply{}, plan_final{};
    const GemmTile sym_tile = plan_tiles(gp, plan_gram, true, ws, kStageGram);
    const GemmTile poly_tile = plan_tiles(gp, plan_poly, true, ws, kStagePoly);
    const GemmTile apply_tile = plan_tiles(gp, plan_apply, false, ws, kStageApply);
    plan_tiles(gp, plan_final, false, nullptr, kStageApply);  // the last Apply keeps every tile whole
    for (int it = 0; it < hp.ns_steps; ++it) {
        const int cur = it & 1, nxt = cur ^ 1;
        const bool last = it + 1 == hp.ns_steps;
        na.first = it == 0 ? 1 : 0;
        for (int k = 0; k < ng; ++k) {
            const MatPlan& p = gp.mats[k];
            NsDesc& d = na.d[k];
            d.xr = reinterpret_cast<const unsigned short*>(ws + p.xr[cur]);
            d.xc = reinterpret_cast<const unsigned short*>(ws + p.xc[cur]);
            d.xr_next = need_xr ? reinterpret_cast<unsigned short*>(ws + p.xr[nxt]) : nullptr;
            d.xc_next = reinterpret_cast<unsigned short*>(ws + p.xc[nxt]);
            d.a = reinterpret_cast<unsigned short*>(ws + p.a);
            d.b = reinterpret_cast<unsigned short*>(ws + p.b);
            d.out = (last && eq6) ? reinterpret_cast<float*>(ws + p.xr[0]) : io[k].out;
            d.part = (last && (eq6 || monitor)) ? reinterpret_cast<float*>(ws + p.rpart) : nullptr;
            d.scale = reinterpret_cast<const float*>(ws + p.scale);
            d.m = int32_t(p.m);
            d.n = int32_t(p.n);
            d.m_p = int32_t(p.m_p);
            d.n_p = int32_t(p.n_p);
            d.tall = p.tall ? 1 : 0;
            d.upd_coef = float(double(hp.lr) * dir_scale(hp, p.n));
        }
        take_tiling(na, plan_gram, ng);
        rc = run_kernel(MUON_KCLASS_GRAM, s, "gram", [&] { return launch_ns_gemm(kModeGram, sym_tile, na, s); });
        if (rc) return rc;
        take_tiling(na, plan_poly, ng);
        rc = run_kernel(MUON_KCLASS_POLY, s, "poly", [&] { return launch_ns_gemm(kModePoly, poly_tile, na, s); });
        if (rc) return rc;
        take_tiling(na, last ? plan_final : plan_apply, ng);
        const GemmMode mode = !last ? kModeApply : ((update_w && !eq6) ? kModeFinalW : kModeFinalO);
        rc = run_kernel(last ? MUON_KCLASS_APPLY_FINAL : MUON_KCLASS_APPLY, s, "apply",
                        [&] { return launch_ns_gemm(mode, apply_tile, na, s); });
        if (rc) return rc;
    }
    if (eq6 || monitor) {
        RmsArgs ra{};
        ra.n = ng;
        ra.lr = hp.lr;
        ra.rms_scale = hp.rms_scale;
        ra.eps = hp.eps;
        for (int k = 0; k < ng; ++k) {
            const MatPlan& p = gp.mats[k];
            RmsDesc& r = ra.d[k];
            r.part = reinterpret_cast<const float*>(ws + p.rpart);
            r.count = na.d[k].ntiles * 4;  // the final apply's tiles, four waves each
            r.elems = double(p.rows) * double(p.cols);
            r.dir_scale = float(dir_scale(hp, p.n));
            r.eq6 = eq6 ? 1 : 0;
            r.coef_out = eq6 ? reinterpret_cast<float*>(ws + p.coef) : nullptr;
            r.rms_out = update_rms ? update_rms + p.idx : nullptr;
        }
        rc = run_kernel(MUON_KCLASS_RMS_FINALIZE, s, "rms_finalize", [&] { return launch_rms_finalize(ra, s); });
        if (rc) return rc;
    }
    if (eq6) {
        UpdArgs ua{};
        ua.n = ng;
        ua.decay = na.decay;
        int64_t blocks = 0;
        for (int k = 0; k < ng; ++k) {
            const MatPlan& p = gp.mats[k];
            UpdDesc& u = ua.d[k];
            u.o = reinterpret_cast<const float*>(ws + p.xr[0]);
            u.w = io[k].out;
            u.coef = reinterpret_cast<const float*>(ws + p.coef);
            u.elems = p.rows * p.cols;
            u.blk_begin = int32_t(blocks);
            blocks += (u.elems + kUpdBlockElems - 1) / kUpdBlockElems;
        }
        ua.total = int32_t(blocks);
        rc = run_kernel(MUON_KCLASS_SCALED_UPDATE, s, "scaled_update", [&] { return launch_scaled_update(ua, s); });
        if (rc) return rc;
    }
    return MUON_OK;
}

int run_rownorm(const GroupPlan& gp, const muon_matrix* mats, const muon_hparams& hp, char* ws,
                float* update_rms, hipStream_t s) {
    const float decay = 1.0f - hp.lr * hp.weight_decay;
    RowArgs ra{}, rw{};  // flat rows; wide flat rows (kRowWideCols < cols <= kRowMaxRegisterCols, cols % 4 == 0)
    ra.mu = rw.mu = hp.mu;
    ra.decay = rw.decay = decay;
    ra.eps = rw.eps = hp.eps;
    ColArgs ca{};
    ca.mu = hp.mu;
    ca.decay = decay;
    ca.eps = hp.eps;
    int64_t rows_total = 0, wide_total = 0, col_total = 0, fin_total = 0;
    int max_cols = 0, max_wide = 0;
    bool row_vec = true, col_vec = true;
    for (const MatPlan& p : gp.mats) {
        const muon_matrix& t = mats[p.idx];
        const float coef = float(double(hp.lr) * double(hp.gamma) * dir_scale(hp, p.n));
        float* part = update_rms ? reinterpret_cast<float*>(ws + p.rpart_rn) : nullptr;
        if (!p.tall) {
            const bool wide = p.cols > kRowWideCols && p.cols <= kRowMaxRegisterCols && p.cols % 4 == 0;
            RowArgs& a = wide ? rw : ra;
            int64_t& total = wide ? wide_total : rows_total;
            RowDesc& d = a.d[a.n++];
            d.g = t.g;
            d.m = t.m;
            d.w = t.w;
            d.rows = int32_t(p.rows);
            d.cols = int32_t(p.cols);
            d.row_begin = int32_t(total);
            d.coef = coef;
            d.part = part;
            total += p.rows;
            if (wide) {
                max_wide = std::max<int>(max_wide, int(p.cols));
            } else {
                max_cols = std::max<int>(max_cols, int(p.cols));
                row_vec = row_vec && (p.cols % 4 == 0);
            }
        } else {
            ColDesc& d = ca.d[ca.n++];
            d.g = t.g;
            d.m = t.m;
            d.w = t.w;
            d.partial = reinterpret_cast<float*>(ws + p.colpart);
            d.inv = reinterpret_cast<float*>(ws + p.inv);
            d.rows = int32_t(p.rows);
            d.cols = int32_t(p.cols);
            d.chunks = int32_t(p.chunks);
            d.tiles_c = int32_t((p.cols + kColTileCols - 1) / kColTileCols);
            d.tile_begin = int32_t(col_total);
            d.fin_begin = int32_t(fin_total);
            d.coef = coef;
            d.part = part;
            col_total += int64_t(d.chunks) * d.tiles_c;
            fin_total += (p.cols + kColFinCols - 1) / kColFinCols;
            col_vec = col_vec && (p.cols % 4 == 0);
        }
    }
    int rc = MUON_OK;
    if (rw.n > 0) {
        rw.total = int32_t(wide_total);
        rc = run_kernel(MUON_KCLASS_ROWNORM_ROWS, s, "rownorm_rows_wide",
                        [&] { return launch_rownorm_rows_wide(rw, max_wide, s); });
        if (rc) return rc;
    }
    if (ra.n > 0) {
        ra.total = int32_t(rows_total);
        rc = run_kernel(MUON_KCLASS_ROWNORM_ROWS, s, "rownorm_rows",
                        [&] { return launch_rownorm_rows(ra, max_cols, row_vec, s); });
        if (rc) return rc;
    }
    if (ca.n > 0) {
        ca.total = int32_t(col_total);
        rc = run_kernel(MUON_KCLASS_COLNORM_PARTIAL, s, "colnorm_partial",
                        [&] { return launch_colnorm_partial(ca, col_vec, s); });
        if (rc) return rc;
        rc = run_kernel(MUON_KCLASS_COLNORM_FINALIZE, s, "colnorm_finalize",
                        [&] { return launch_colnorm_finalize(ca, int(fin_total), s); });
        if (rc) return rc;
        rc = run_kernel(MUON_KCLASS_COLNORM_APPLY, s, "colnorm_apply",
                        [&] { return launch_colnorm_apply(ca, col_vec, s); });
        if (rc) return rc;
    }
    if (update_rms) {
        RmsArgs ra{};
        ra.n = int32_t(gp.mats.size());
        ra.lr = hp.lr;
        ra.rms_scale = hp.rms_scale;
        ra.eps = hp.eps;
        for (int k = 0; k < ra.n; ++k) {
            const MatPlan& p = gp.mats[k];
            RmsDesc& r = ra.d[k];
            r.part = reinterpret_cast<const float*>(ws + p.rpart_rn);
            r.count = int32_t(p.tall ? p.cols : p.rows);
            r.elems = double(p.rows) * double(p.cols);
            r.dir_scale = float(double(hp.gamma) * dir_scale(hp, p.n));
            r.eq6 = 0;
            r.coef_out = nullptr;
            r.rms_out = update_rms + p.idx;
        }
        rc = run_kernel(MUON_KCLASS_RMS_FINALIZE, s, "rms_finalize", [&] { return launch_rms_finalize(ra, s); });
    }
    return rc;
}

int do_rownorm(const muon_matrix* mats, int32_t count, const muon_hparams* hp, void* ws,
               size_t ws_bytes, float* update_rms, void* stream, bool need_k) {
    g_last_error.clear();
    int rc = check_hparams(hp, need_k);
    if (rc) return rc;
    std::vector<int64_t> rows, cols;
    std::vector<Range> ranges;
    rc = check_matrices(mats, count, rows, cols, ranges);
    if (rc) return rc;
    rc = check_monitor(update_rms, count, ranges);
    if (rc) return rc;
    Plan plan;
    rc = make_plan(rows.data(), cols.data(), count, &plan);
    if (rc) return rc;
    rc = check_workspace(plan, ws, ws_bytes, ranges);
    if (rc) return rc;
    rc = check_overlaps(ranges);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (const GroupPlan& gp : plan.groups) {
        rc = run_rownorm(gp, mats, *hp, static_cast<char*>(ws), update_rms, s);
        if (rc) return rc;
    }
    return MUON_OK;
}

// ------------------------------------------------- row-sharded RowNorm share ----
// One GPU's share of the RowNorm step of a tall matrix sharded by rows ([DiT]
// distributed-implementation paragraph): the block's momentum update and column sums
// of M'^2 (rownorm_shard_colsq), then, with the totals the caller reduced across the
// GPUs, the column-normalised update (rownorm_shard_apply). Both reuse the tall RowNorm
// kernels; the workspace holds per-shard chunk partials and inverse norms.
struct ShardPlan {
    int idx;
    int64_t rows, cols, chunks;
    size_t partial, inv;  // workspace offsets relative to the group base
};

int plan_shards(const muon_shard* shards, int32_t count, std::vector<std::vector<ShardPlan>>* groups,
                size_t* bytes) {
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && !shards) return fail(MUON_ERR_INVALID_ARG, "shards is NULL");
    *bytes = 0;
    std::vector<ShardPlan> cur;
    size_t off = 0;
    for (int i = 0; i < count; ++i) {
        const muon_shard& t = shards[i];
        if (t.rows < 0 || t.cols < 0 || t.full_rows < 0)
            return fail(MUON_ERR_INVALID_ARG, "negative dimension at index " + std::to_string(i));
        if (t.cols == 0) continue;
        if (t.rows > kMaxDim || t.cols > kMaxDim || t.full_rows > kMaxDim || t.rows * t.cols > kMaxElems)
            return fail(MUON_ERR_TOO_LARGE, "shard " + std::to_string(i) + " too large");
        if (t.full_rows <= t.cols)
            return fail(MUON_ERR_INVALID_ARG, "shard " + std::to_string(i) +
                                                  ": full_rows must exceed cols (flat matrices use rownorm_update)");
        if (t.rows > t.full_rows)
            return fail(MUON_ERR_INVALID_ARG, "shard " + std::to_string(i) + ": rows above full_rows");
        if (cur.size() == size_t(kMaxGroup)) {
            groups->push_back(std::move(cur));
            cur.clear();
            *bytes = std::max(*bytes, off);
            off = 0;
        }
        ShardPlan sp{};
        sp.idx = i;
        sp.rows = t.rows;
        sp.cols = t.cols;
        sp.chunks = (t.rows + kColChunkRows - 1) / kColChunkRows;
        sp.partial = off;
        off += align256(size_t(std::max<int64_t>(sp.chunks, 1)) * size_t(t.cols) * 4);
        sp.inv = off;
        off += align256(size_t(t.cols) * 4);
        cur.push_back(sp);
    }
    if (!cur.empty()) {
        groups->push_back(std::move(cur));
        *bytes = std::max(*bytes, off);
    }
    return MUON_OK;
}

// Validates pointers, alignment and overlaps of a shard call; `sums` are the caller's
// per-shard column-sum arrays (written by colsq, read by apply).
int check_shard_buffers(const muon_shard* shards, const std::vector<std::vector<ShardPlan>>& groups,
                        const float* const* sums, bool sums_written, bool need_g, size_t need_bytes, void* ws,
                        size_t ws_bytes, std::vector<Range>& ranges) {
    if (groups.empty()) return MUON_OK;
    if (!sums) return fail(MUON_ERR_INVALID_ARG, "column-sum array is NULL");
    for (const auto& g : groups)
        for (const ShardPlan& sp : g) {
            const muon_shard& t = shards[sp.idx];
            const std::string at = " at index " + std::to_string(sp.idx);
            const float* cs = sums[sp.idx];
            if (!cs) return fail(MUON_ERR_INVALID_ARG, "NULL column sums" + at);
            if (reinterpret_cast<uintptr_t>(cs) & 3) return fail(MUON_ERR_ALIGN, "column sums not 4-byte aligned" + at);
            const uintptr_t lo = reinterpret_cast<uintptr_t>(cs);
            ranges.push_back({lo, lo + uintptr_t(sp.cols) * 4, sums_written});
            if (sp.rows == 0) continue;
            if (!t.w || !t.m || (need_g && !t.g)) return fail(MUON_ERR_INVALID_ARG, "NULL pointer" + at);
            if (!aligned16(t.w) || !aligned16(t.m) || (t.g && !aligned16(t.g)))
                return fail(MUON_ERR_ALIGN, "matrix pointer not 16-byte aligned" + at);
            const uintptr_t bytes = uintptr_t(sp.rows * sp.cols) * 4;
            ranges.push_back({reinterpret_cast<uintptr_t>(t.w), reinterpret_cast<uintptr_t>(t.w) + bytes, true});
            ranges.push_back({reinterpret_cast<uintptr_t>(t.m), reinterpret_cast<uintptr_t>(t.m) + bytes, true});
            if (need_g)
                ranges.push_back({reinterpret_cast<uintptr_t>(t.g), reinterpret_cast<uintptr_t>(t.g) + bytes, false});
        }
    if (!ws) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if (ws_bytes < need_bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need_bytes) + " bytes");
    if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MUON_ERR_ALIGN, "workspace not 256-byte aligned");
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ws);
    ranges.push_back({lo, lo + need_bytes, true});
    return check_overlaps(ranges);
}

// ------------------------------------------------------ singular spectrum ----
// SVD-entropy diagnostic ("Muon is Scalable", Sec. 3.4). Per matrix: the fp64 Gram
// matrix S (m_p x m_p), seven m_p vectors (v_j twice, w, p, d, e, eigenvalues), the
// pass kernel's two partial arrays (tp x tp tiles of 64 doubles, tp = m_p / 64) and
// tau; groups of up to kMaxGroup matrices (largest m first) share one workspace
// region and run one after another.
constexpr int64_t kSpMaxM = 65536;

struct SpMat {
    int idx;
    int64_t rows, cols;
    int32_t m, n, tm;
    bool tall;
    int64_t m_p;
    size_t off;          // workspace offset relative to the group base
    int64_t sigma_off;   // offset into the caller's sigma_sq array
};

struct SpPlan {
    std::vector<std::vector<SpMat>> groups;
    size_t bytes = 0;
    int64_t sigma_total = 0;
};

size_t sp_vec_bytes(int64_t m_p) { return align256(size_t(m_p) * 8); }
size_t sp_part_bytes(int64_t m_p) {
    const size_t tp = size_t(m_p / kSpPassTile);
    return align256(tp * tp * kSpPassTile * 8);
}
size_t sp_mat_bytes(int64_t m_p) {
    return align256(size_t(m_p) * size_t(m_p) * 8) + 7 * sp_vec_bytes(m_p) + 2 * sp_part_bytes(m_p) + 256;
}

int make_sp_plan(const int64_t* rows, const int64_t* cols, int32_t count, SpPlan* plan) {
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "rows or cols is NULL");
    std::vector<SpMat> mats;
    for (int i = 0; i < count; ++i) {
        const int64_t r = rows[i], c = cols[i];
        if (r < 0 || c < 0) return fail(MUON_ERR_INVALID_ARG, "negative dimension at index " + std::to_string(i));
        if (r == 0 || c == 0) continue;
        if (r > kMaxDim || c > kMaxDim || r * c > kMaxElems)
            return fail(MUON_ERR_TOO_LARGE, "matrix " + std::to_string(i) + " too large");
        if (std::min(r, c) > kSpMaxM)
            return fail(MUON_ERR_TOO_LARGE, "matrix " + std::to_string(i) + ": min(rows, cols) above 65536");
        SpMat sm{};
        sm.idx = i;
        sm.rows = r;
        sm.cols = c;
        sm.tall = r > c;
        sm.m = int32_t(std::min(r, c));
        sm.n = int32_t(std::max(r, c));
        sm.m_p = round_up(sm.m, kSpTile);
        sm.tm = int32_t(sm.m_p / kSpTile);
        sm.sigma_off = plan->sigma_total;
        plan->sigma_total += sm.m;
        mats.push_back(sm);
    }
    std::stable_sort(mats.begin(), mats.end(), [](const SpMat& a, const SpMat& b) { return a.m > b.m; });
    for (size_t k = 0; k < mats.size(); k += kMaxGroup) {
        std::vector<SpMat> g(mats.begin() + k, mats.begin() + std::min(mats.size(), k + kMaxGroup));
        size_t off = 0;
        for (SpMat& sm : g) {
            sm.off = off;
            off += sp_mat_bytes(sm.m_p);
        }
        plan->bytes = std::max(plan->bytes, off);
        plan->groups.push_back(std::move(g));
    }
    return MUON_OK;
}

int run_spectrum(const std::vector<SpMat>& g, const float* const* w, char* ws, double* entropy,
                 double* sigma_sq, hipStream_t s) {
    SpArgs a{};
    a.n = int32_t(g.size());
    a.sigma_sq = sigma_sq;
    int32_t tiles = 0, max_m = 0;
    for (int k = 0; k < a.n; ++k) {
        const SpMat& sm = g[k];
        SpDesc& d = a.d[k];
        d.w = w[sm.idx];
        d.cols = sm.cols;
        d.m = sm.m;
        d.n = sm.n;
        d.tall = sm.tall ? 1 : 0;
        d.tm = sm.tm;
        d.tile_begin = tiles;
        d.sigma_off = sm.sigma_off;
        d.ld = sm.m_p;
        char* base = ws + sm.off;
        d.s = reinterpret_cast<double*>(base);
        base += align256(size_t(sm.m_p) * size_t(sm.m_p) * 8);
        double** vecs[7] = {&d.v[0], &d.v[1], &d.wv, &d.p, &d.d, &d.e, &d.lam};
        for (double** v : vecs) {
            *v = reinterpret_cast<double*>(base);
            base += sp_vec_bytes(sm.m_p);
        }
        d.rowpart = reinterpret_cast<double*>(base);
        base += sp_part_bytes(sm.m_p);
        d.colpart = reinterpret_cast<double*>(base);
        base += sp_part_bytes(sm.m_p);
        d.tp = int32_t(sm.m_p / kSpPassTile);
        d.tau = reinterpret_cast<double*>(base);
        d.entropy = entropy + sm.idx;
        tiles += sm.tm * (sm.tm + 1) / 2;
        max_m = std::max(max_m, sm.m);
    }
    a.total = tiles;
    int rc = run_kernel(MUON_KCLASS_SPEC_GRAM, s, "spectrum gram", [&] { return launch_sp_gram(a, s); });
    if (rc) return rc;
    for (int j = 0; j < max_m; ++j) {
        a.j = j;
        rc = run_kernel(MUON_KCLASS_SPEC_HOUSE, s, "spectrum house", [&] { return launch_sp_house(a, s); });
        if (rc) return rc;
        if (j <= max_m - 2) {
            int max_tiles = 0;
            for (const SpMat& sm : g) {
                if (j > sm.m - 2) continue;
                const int nt = (sm.m + kSpPassTile - 1) / kSpPassTile - (j + 1) / kSpPassTile;
                max_tiles = std::max(max_tiles, nt * (nt + 1) / 2);
            }
            rc = run_kernel(MUON_KCLASS_SPEC_PASS, s, "spectrum pass",
                            [&] { return launch_sp_pass(a, max_tiles, s); });
            if (rc) return rc;
            rc = run_kernel(MUON_KCLASS_SPEC_REDUCE, s, "spectrum reduce",
                            [&] { return launch_sp_reduce(a, max_m - j - 1, s); });
            if (rc) return rc;
        }
    }
    rc = run_kernel(MUON_KCLASS_SPEC_BISECT, s, "spectrum bisect", [&] { return launch_sp_bisect(a, max_m, s); });
    if (rc) return rc;
    return run_kernel(MUON_KCLASS_SPEC_ENTROPY, s, "spectrum entropy", [&] { return launch_sp_entropy(a, s); });
}

}  // namespace

int set_last_error(int code, const std::string& what) { return fail(code, what); }

// The RowNorm step on a scratch buffer the library holds (the allocation-free entry
// point, csrc/noalloc.hip). Every argument is validated and the step planned on the
// host first; only then, and only when there is work, does get_scratch fetch the
// current device's scratch address. Groups run one after another on the same region,
// as with a caller's workspace; every scratch element a kernel reads was written
// earlier in the same call, so nothing has to start at zero. No event is created
// for the timing facility.
int rownorm_noalloc_impl(const muon_matrix* mats, int32_t count, const muon_hparams* hp, float* update_rms,
                         void* stream, size_t scratch_cap, void* (*get_scratch)(std::string* error)) {
    g_last_error.clear();
    int rc = check_hparams(hp, false);
    if (rc) return rc;
    std::vector<int64_t> rows, cols;
    std::vector<Range> ranges;
    rc = check_matrices(mats, count, rows, cols, ranges);
    if (rc) return rc;
    rc = check_monitor(update_rms, count, ranges);
    if (rc) return rc;
    Plan plan;
    rc = make_plan(rows.data(), cols.data(), count, &plan);
    if (rc) return rc;
    if (plan.rn_bytes > scratch_cap)
        return fail(MUON_ERR_WORKSPACE, "these matrices need " + std::to_string(plan.rn_bytes) +
                                            " bytes of scratch; the library's fixed scratch holds " +
                                            std::to_string(scratch_cap) + " (call rownorm_update with a workspace)");
    rc = check_overlaps(ranges);
    if (rc) return rc;
    if (plan.groups.empty()) return MUON_OK;
    std::string err;
    char* ws = static_cast<char*>(get_scratch(&err));
    if (!ws) return fail(MUON_ERR_HIP, "scratch address: " + err);
    const uintptr_t lo = reinterpret_cast<uintptr_t>(ws);
    ranges.push_back({lo, lo + plan.rn_bytes, true});
    rc = check_overlaps(ranges);  // a caller's buffer inside the library's scratch
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    ++g_untimed;
    for (const GroupPlan& gp : plan.groups) {
        rc = run_rownorm(gp, mats, *hp, ws, update_rms, s);
        if (rc) break;
    }
    --g_untimed;
    return rc;
}

}  // namespace muon

using namespace muon;

MUON_API int muon_abi_version(void) { return MUON_ABI_VERSION; }

MUON_API const char* muon_status_str(int status) {
    switch (status) {
        case MUON_OK: return "ok";
        case MUON_ERR_INVALID_ARG: return "invalid argument";
        case MUON_ERR_WORKSPACE: return "workspace missing or too small";
        case MUON_ERR_ALIGN: return "misaligned pointer";
        case MUON_ERR_ALIAS: return "overlapping buffers";
        case MUON_ERR_HIP: return "HIP runtime error";
        case MUON_ERR_TOO_LARGE: return "problem too large";
        default: return "unknown status";
    }
}

MUON_API const char* muon_last_error(void) { return g_last_error.c_str(); }

MUON_API void muon_default_hparams(muon_hparams* hp) {
    if (!hp) return;
    hp->lr = 1e-3f;
    hp->weight_decay = 0.1f;
    hp->mu = 0.95f;
    hp->ns_a = 3.4445f;
    hp->ns_b = -4.7750f;
    hp->ns_c = 2.0315f;
    hp->rms_scale = 0.2f;
    hp->gamma = 0.15f;
    hp->eps = 1e-7f;
    hp->ns_steps = 5;
    hp->period_k = 3;
    hp->scale_mode = MUON_SCALE_MAX_DIM;
    hp->hidden = 0;
}

MUON_API int muon_workspace_bytes(const int64_t* rows, const int64_t* cols, int32_t count, size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "rows or cols is NULL");
    Plan plan;
    const int rc = make_plan(rows, cols, count, &plan);
    if (rc) return rc;
    *bytes = plan.bytes;
    return MUON_OK;
}

MUON_API int ns5_plan(const int64_t* rows, const int64_t* cols, int32_t count, int32_t* out, int32_t capacity,
                      int32_t* groups) {
    g_last_error.clear();
    if (!groups) return fail(MUON_ERR_INVALID_ARG, "groups is NULL");
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "rows or cols is NULL");
    if (capacity < 0 || (capacity > 0 && !out)) return fail(MUON_ERR_INVALID_ARG, "out is NULL or capacity < 0");
    Plan plan;
    const int rc = make_plan(rows, cols, count, &plan);
    if (rc) return rc;
    const int64_t ng = int64_t(plan.groups.size());
    *groups = int32_t(ng);
    if (capacity == 0) return MUON_OK;
    if (ng * MUON_PLAN_RECORD_INTS > capacity)
        return fail(MUON_ERR_INVALID_ARG, "capacity holds fewer than groups x MUON_PLAN_RECORD_INTS values");
    static_assert(MUON_PLAN_RECORD_INTS == 1 + kMaxGroup + 4 * 17, "plan record layout");
    for (int64_t g = 0; g < ng; ++g) {
        const GroupPlan& gp = plan.groups[size_t(g)];
        int32_t* r = out + g * MUON_PLAN_RECORD_INTS;
        r[0] = int32_t(gp.mats.size());
        for (int k = 0; k < kMaxGroup; ++k) r[1 + k] = k < int(gp.mats.size()) ? int32_t(gp.mats[size_t(k)].idx) : -1;
        // Gram, polynomial, Apply of iterations 1..N-1, last Apply: as run_refresh plans them
        const bool sym[4] = {true, true, false, false};
        const int stage[4] = {kStageGram, kStagePoly, kStageApply, kStageApply};
        const bool split[4] = {true, true, true, false};
        for (int st = 0; st < 4; ++st) {
            NsArgs na{};
            bool head = false;
            const GemmTile tile = plan_tiles(gp, na, sym[st], nullptr, stage[st], split[st], &head);
            int32_t* q = r + 1 + kMaxGroup + st * 17;
            q[0] = tile == kTileBig ? int32_t(kGemmBigM) : int32_t(kGemmSmall);
            for (int x = 0; x < 8; ++x) {
                q[1 + 2 * x] = na.fix_total > 0 ? (head ? -na.xtail[x] : na.xtail[x]) : 0;
                q[2 + 2 * x] = na.fix_total > 0 ? na.xsplit[x] : 1;
            }
        }
    }
    return MUON_OK;
}

MUON_API int muon_step(const muon_matrix* mats, int32_t count, const muon_hparams* hp, int64_t step,
                       void* workspace, size_t workspace_bytes, float* update_rms, void* stream) {
    g_last_error.clear();
    if (step < 0) return fail(MUON_ERR_INVALID_ARG, "step < 0");
    int rc = check_hparams(hp, true);
    if (rc) return rc;
    if (step % hp->period_k != 0)
        return do_rownorm(mats, count, hp, workspace, workspace_bytes, update_rms, stream, true);
    std::vector<int64_t> rows, cols;
    std::vector<Range> ranges;
    rc = check_matrices(mats, count, rows, cols, ranges);
    if (rc) return rc;
    rc = check_monitor(update_rms, count, ranges);
    if (rc) return rc;
    Plan plan;
    rc = make_plan(rows.data(), cols.data(), count, &plan);
    if (rc) return rc;
    rc = check_workspace(plan, workspace, workspace_bytes, ranges);
    if (rc) return rc;
    rc = check_overlaps(ranges);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (const GroupPlan& gp : plan.groups) {
        std::vector<IoPtrs> io;
        for (const MatPlan& p : gp.mats) {
            const muon_matrix& t = mats[p.idx];
            io.push_back({t.m, t.g, t.m, t.w});
        }
        rc = run_refresh(gp, io, *hp, true, true, static_cast<char*>(workspace), update_rms, s);
        if (rc) return rc;
    }
    return MUON_OK;
}

MUON_API int ns5_batched(const float* const* m_in, float* const* o_out, const int64_t* rows,
                         const int64_t* cols, int32_t count, const muon_hparams* hp, void* workspace,
                         size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    int rc = check_hparams(hp, false);
    if (rc) return rc;
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && (!m_in || !o_out || !rows || !cols))
        return fail(MUON_ERR_INVALID_ARG, "NULL array argument");
    std::vector<Range> ranges;
    for (int i = 0; i < count; ++i) {
        if (rows[i] < 0 || cols[i] < 0) return fail(MUON_ERR_INVALID_ARG, "negative dimension at index " + std::to_string(i));
        if (rows[i] == 0 || cols[i] == 0) continue;
        if (rows[i] > kMaxDim || cols[i] > kMaxDim || rows[i] * cols[i] > kMaxElems)
            return fail(MUON_ERR_TOO_LARGE, "matrix " + std::to_string(i) + " exceeds the size limits");
        if (!m_in[i] || !o_out[i]) return fail(MUON_ERR_INVALID_ARG, "NULL matrix pointer at index " + std::to_string(i));
        if (!aligned16(m_in[i]) || !aligned16(o_out[i]))
            return fail(MUON_ERR_ALIGN, "matrix pointer not 16-byte aligned at index " + std::to_string(i));
        const uintptr_t bytes = uintptr_t(rows[i]) * uintptr_t(cols[i]) * 4;
        const uintptr_t pi = reinterpret_cast<uintptr_t>(m_in[i]), po = reinterpret_cast<uintptr_t>(o_out[i]);
        if (pi == po) {
            ranges.push_back({po, po + bytes, true});
        } else {
            ranges.push_back({pi, pi + bytes, false});
            ranges.push_back({po, po + bytes, true});
        }
    }
    Plan plan;
    rc = make_plan(rows, cols, count, &plan);
    if (rc) return rc;
    rc = check_workspace(plan, workspace, workspace_bytes, ranges);
    if (rc) return rc;
    rc = check_overlaps(ranges);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (const GroupPlan& gp : plan.groups) {
        std::vector<IoPtrs> io;
        for (const MatPlan& p : gp.mats) io.push_back({m_in[p.idx], nullptr, nullptr, o_out[p.idx]});
        rc = run_refresh(gp, io, *hp, false, false, static_cast<char*>(workspace), nullptr, s);
        if (rc) return rc;
    }
    return MUON_OK;
}

MUON_API int rownorm_update(const muon_matrix* mats, int32_t count, const muon_hparams* hp,
                            void* workspace, size_t workspace_bytes, float* update_rms, void* stream) {
    return do_rownorm(mats, count, hp, workspace, workspace_bytes, update_rms, stream, false);
}

MUON_API void adamw_default_hparams(adamw_hparams* hp) {
    if (!hp) return;
    hp->lr = 1e-4f;
    hp->beta1 = 0.9f;
    hp->beta2 = 0.999f;
    hp->eps = 1e-8f;
    hp->weight_decay = 0.1f;
}

MUON_API int adamw_step(const adamw_param* params, int32_t count, const adamw_hparams* hp, int64_t step,
                        void* stream) {
    g_last_error.clear();
    if (!hp) return fail(MUON_ERR_INVALID_ARG, "hparams is NULL");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return fail(MUON_ERR_INVALID_ARG, "lr and weight_decay must be finite");
    if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f) || !(hp->beta2 >= 0.f && hp->beta2 < 1.f))
        return fail(MUON_ERR_INVALID_ARG, "beta1 and beta2 must be in [0, 1)");
    if (!(hp->eps > 0.f) || !std::isfinite(hp->eps)) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (step < 0) return fail(MUON_ERR_INVALID_ARG, "step < 0");
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
    if (count > 0 && !params) return fail(MUON_ERR_INVALID_ARG, "params is NULL");
    std::vector<Range> ranges;
    for (int i = 0; i < count; ++i) {
        const adamw_param& p = params[i];
        if (p.numel < 0) return fail(MUON_ERR_INVALID_ARG, "negative numel at index " + std::to_string(i));
        if (p.numel == 0) continue;
        if (p.numel > kMaxElems) return fail(MUON_ERR_TOO_LARGE, "tensor " + std::to_string(i) + " above 2^40 elements");
        if (!p.w || !p.m || !p.v || !p.g) return fail(MUON_ERR_INVALID_ARG, "NULL pointer at index " + std::to_string(i));
        if (!aligned16(p.w) || !aligned16(p.m) || !aligned16(p.v) || !aligned16(p.g))
            return fail(MUON_ERR_ALIGN, "tensor pointer not 16-byte aligned at index " + std::to_string(i));
        const uintptr_t bytes = uintptr_t(p.numel) * 4;
        ranges.push_back({reinterpret_cast<uintptr_t>(p.w), reinterpret_cast<uintptr_t>(p.w) + bytes, true});
        ranges.push_back({reinterpret_cast<uintptr_t>(p.m), reinterpret_cast<uintptr_t>(p.m) + bytes, true});
        ranges.push_back({reinterpret_cast<uintptr_t>(p.v), reinterpret_cast<uintptr_t>(p.v) + bytes, true});
        ranges.push_back({reinterpret_cast<uintptr_t>(p.g), reinterpret_cast<uintptr_t>(p.g) + bytes, false});
    }
    int rc = check_overlaps(ranges);
    if (rc) return rc;
    // bias corrections in double on the host (t = step + 1)
    const double t = double(step) + 1.0;
    const double bc1 = 1.0 - std::pow(double(hp->beta1), t);
    const double bc2 = 1.0 - std::pow(double(hp->beta2), t);
    AdamArgs a{};
    a.beta1 = hp->beta1;
    a.beta2 = hp->beta2;
    a.one_minus_beta1 = float(1.0 - double(hp->beta1));
    a.one_minus_beta2 = float(1.0 - double(hp->beta2));
    a.eps = hp->eps;
    a.decay = float(1.0 - double(hp->lr) * double(hp->weight_decay));
    a.lr_bc1 = float(double(hp->lr) / bc1);
    a.inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int64_t blocks = 0;
    auto flush = [&]() -> int {
        if (a.n == 0) return MUON_OK;
        a.total = int32_t(blocks);
        const int r = run_kernel(MUON_KCLASS_ADAMW, s, "adamw", [&] { return launch_adamw(a, s); });
        a.n = 0;
        blocks = 0;
        return r;
    };
    for (int i = 0; i < count; ++i) {
        const adamw_param& p = params[i];
        if (p.numel == 0) continue;
        const int64_t nb = (p.numel + kAdamBlockElems - 1) / kAdamBlockElems;
        if (a.n == kAdamMaxTensors || blocks + nb >= (int64_t(1) << 31)) {
            rc = flush();
            if (rc) return rc;
        }
        AdamDesc& d = a.d[a.n++];
        d.w = p.w;
        d.m = p.m;
        d.v = p.v;
        d.g = p.g;
        d.n = p.numel;
        d.blk_begin = int32_t(blocks);
        blocks += nb;
    }
    return flush();
}

MUON_API int rownorm_shard_workspace_bytes(const muon_shard* shards, int32_t count, size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
    std::vector<std::vector<ShardPlan>> groups;
    return plan_shards(shards, count, &groups, bytes);
}

MUON_API int rownorm_shard_colsq(const muon_shard* shards, int32_t count, const muon_hparams* hp,
                                 float* const* colsq, void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    int rc = check_hparams(hp, false);
    if (rc) return rc;
    std::vector<std::vector<ShardPlan>> groups;
    size_t need = 0;
    rc = plan_shards(shards, count, &groups, &need);
    if (rc) return rc;
    std::vector<Range> ranges;
    rc = check_shard_buffers(shards, groups, colsq, true, true, need, workspace, workspace_bytes, ranges);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    for (const auto& g : groups) {
        ColArgs ca{};
        ca.mu = hp->mu;
        ca.eps = hp->eps;
        ca.sums_only = 1;
        int64_t tiles = 0, fin = 0;
        for (const ShardPlan& sp : g) {
            const muon_shard& t = shards[sp.idx];
            ColDesc& d = ca.d[ca.n++];
            d.g = t.g;
            d.m = t.m;
            d.partial = reinterpret_cast<float*>(ws + sp.partial);
            d.inv = colsq[sp.idx];
            d.rows = int32_t(sp.rows);
            d.cols = int32_t(sp.cols);
            d.chunks = int32_t(sp.chunks);  // 0 for an empty block: its sums are written as 0
            d.tiles_c = int32_t((sp.cols + kColTileCols - 1) / kColTileCols);
            d.tile_begin = int32_t(tiles);
            d.fin_begin = int32_t(fin);
            tiles += int64_t(d.chunks) * d.tiles_c;
            fin += (sp.cols + kColFinCols - 1) / kColFinCols;
        }
        bool vec = true;
        for (const ShardPlan& sp : g) vec = vec && (sp.cols % 4 == 0);
        if (tiles > 0) {
            ca.total = int32_t(tiles);
            rc = run_kernel(MUON_KCLASS_COLNORM_PARTIAL, s, "shard colsq partial",
                            [&] { return launch_colnorm_partial(ca, vec, s); });
            if (rc) return rc;
        }
        rc = run_kernel(MUON_KCLASS_COLNORM_FINALIZE, s, "shard colsq sums",
                        [&] { return launch_colnorm_finalize(ca, int(fin), s); });
        if (rc) return rc;
    }
    return MUON_OK;
}

MUON_API int rownorm_shard_apply(const muon_shard* shards, int32_t count, const muon_hparams* hp,
                                 const float* const* colsq_total, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    g_last_error.clear();
    int rc = check_hparams(hp, false);
    if (rc) return rc;
    std::vector<std::vector<ShardPlan>> groups;
    size_t need = 0;
    rc = plan_shards(shards, count, &groups, &need);
    if (rc) return rc;
    std::vector<Range> ranges;
    rc = check_shard_buffers(shards, groups, colsq_total, false, false, need, workspace, workspace_bytes, ranges);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    const float decay = 1.0f - hp->lr * hp->weight_decay;
    for (const auto& g : groups) {
        ColArgs fa{}, aa{};  // finalize: totals -> 1 / max(norm, eps); apply: the update
        fa.eps = aa.eps = hp->eps;
        fa.decay = aa.decay = decay;
        int64_t tiles = 0, fin = 0;
        for (const ShardPlan& sp : g) {
            const muon_shard& t = shards[sp.idx];
            ColDesc& f = fa.d[fa.n++];
            f.partial = const_cast<float*>(colsq_total[sp.idx]);
            f.inv = reinterpret_cast<float*>(ws + sp.inv);
            f.cols = int32_t(sp.cols);
            f.chunks = 1;
            f.fin_begin = int32_t(fin);
            fin += (sp.cols + kColFinCols - 1) / kColFinCols;
            if (sp.rows == 0) continue;
            ColDesc& d = aa.d[aa.n++];
            d.m = t.m;
            d.w = t.w;
            d.inv = f.inv;
            d.rows = int32_t(sp.rows);
            d.cols = int32_t(sp.cols);
            d.chunks = int32_t(sp.chunks);
            d.tiles_c = int32_t((sp.cols + kColTileCols - 1) / kColTileCols);
            d.tile_begin = int32_t(tiles);
            // the whole matrix's scale: sqrt(max(A, B)) = sqrt(full_rows) for a tall matrix
            d.coef = float(double(hp->lr) * double(hp->gamma) * dir_scale(*hp, t.full_rows));
            tiles += int64_t(d.chunks) * d.tiles_c;
        }
        rc = run_kernel(MUON_KCLASS_COLNORM_FINALIZE, s, "shard inverse norms",
                        [&] { return launch_colnorm_finalize(fa, int(fin), s); });
        if (rc) return rc;
        if (aa.n > 0) {
            bool vec = true;
            for (int k = 0; k < aa.n; ++k) vec = vec && (aa.d[k].cols % 4 == 0);
            aa.total = int32_t(tiles);
            rc = run_kernel(MUON_KCLASS_COLNORM_APPLY, s, "shard apply",
                            [&] { return launch_colnorm_apply(aa, vec, s); });
            if (rc) return rc;
        }
    }
    return MUON_OK;
}

MUON_API int svd_entropy_workspace_bytes(const int64_t* rows, const int64_t* cols, int32_t count,
                                         size_t* bytes) {
    g_last_error.clear();
    if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
    SpPlan plan;
    const int rc = make_sp_plan(rows, cols, count, &plan);
    if (rc) return rc;
    *bytes = plan.bytes;
    return MUON_OK;
}

MUON_API int svd_entropy(const float* const* w, const int64_t* rows, const int64_t* cols, int32_t count,
                         void* workspace, size_t workspace_bytes, double* entropy, double* sigma_sq,
                         void* stream) {
    g_last_error.clear();
    SpPlan plan;
    int rc = make_sp_plan(rows, cols, count, &plan);
    if (rc) return rc;
    if (plan.groups.empty()) return MUON_OK;
    if (!w) return fail(MUON_ERR_INVALID_ARG, "w is NULL");
    if (!entropy) return fail(MUON_ERR_INVALID_ARG, "entropy is NULL");
    if (reinterpret_cast<uintptr_t>(entropy) & 7) return fail(MUON_ERR_ALIGN, "entropy not 8-byte aligned");
    if (sigma_sq && (reinterpret_cast<uintptr_t>(sigma_sq) & 7))
        return fail(MUON_ERR_ALIGN, "sigma_sq not 8-byte aligned");
    std::vector<Range> ranges;
    for (const auto& g : plan.groups)
        for (const SpMat& sm : g) {
            const float* p = w[sm.idx];
            if (!p) return fail(MUON_ERR_INVALID_ARG, "NULL matrix at index " + std::to_string(sm.idx));
            if (!aligned16(p)) return fail(MUON_ERR_ALIGN, "matrix not 16-byte aligned at index " + std::to_string(sm.idx));
            const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
            ranges.push_back({lo, lo + uintptr_t(sm.rows * sm.cols) * 4, false});
        }
    const uintptr_t elo = reinterpret_cast<uintptr_t>(entropy);
    ranges.push_back({elo, elo + uintptr_t(count) * 8, true});
    if (sigma_sq) {
        const uintptr_t slo = reinterpret_cast<uintptr_t>(sigma_sq);
        ranges.push_back({slo, slo + uintptr_t(plan.sigma_total) * 8, true});
    }
    if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if (workspace_bytes < plan.bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(plan.bytes) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(MUON_ERR_ALIGN, "workspace not 256-byte aligned");
    const uintptr_t wlo = reinterpret_cast<uintptr_t>(workspace);
    ranges.push_back({wlo, wlo + plan.bytes, true});
    rc = check_overlaps(ranges);
    if (rc) return rc;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (const auto& g : plan.groups) {
        rc = run_spectrum(g, w, static_cast<char*>(workspace), entropy, sigma_sq, s);
        if (rc) return rc;
    }
    return MUON_OK;
}

MUON_API int muon_timing_enable(int enable) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (!enable) {
        for (TimingRecord& r : g_timing.records) {
            g_timing.pool.push_back(r.start);
            g_timing.pool.push_back(r.stop);
        }
        g_timing.records.clear();
    }
    g_timing.enabled = enable != 0;
    return MUON_OK;
}

MUON_API int muon_timing_read(double* ms, int64_t* launches) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lk(g_timing.mu);
    int rc = MUON_OK;
    for (TimingRecord& r : g_timing.records) {
        float t = 0.f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&t, r.start, r.stop);
        if (e != hipSuccess) {
            rc = fail(MUON_ERR_HIP, std::string("timing: ") + hipGetErrorString(e));
        } else if (r.cls >= 0 && r.cls < MUON_KCLASS_COUNT) {
            if (ms) ms[r.cls] += double(t);
            if (launches) launches[r.cls] += 1;
        }
        g_timing.pool.push_back(r.start);
        g_timing.pool.push_back(r.stop);
    }
    g_timing.records.clear();
    return rc;
}
