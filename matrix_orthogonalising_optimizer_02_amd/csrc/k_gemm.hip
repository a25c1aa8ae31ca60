// Launchers for the Newton-Schulz GEMM stages (kernel body in gemm_kernel.hpp).
//
// Two tile configurations are compiled:
//   small: 128 x 128 block tile, register-staged loads, 64 KiB LDS, 2 blocks per CU;
//   big:   256 x 256 block tile (each wave 128 x 128: half the LDS reads per MFMA of
//          the small tile), K step 32 in a 4-deep ring of LDS stages filled by
//          buffer loads straight to LDS (three K steps of loads in flight), 140 KiB LDS,
//          1 block per CU.
// The host picks, per stage, the big tile when the launch has enough big tiles to
// fill the GPU, and the small one otherwise (small Gram matrices, small sets). A Gram,
// polynomial or non-final Apply stage on big tiles whose XCDs would end on a short last
// round runs those last tiles as K chunks, and a fixup launch adds the chunks and
// applies the epilogue.
#include "gemm_kernel.hpp"

#ifndef MUON_GEMM_BIG_DIRECT
#define MUON_GEMM_BIG_DIRECT 1
#endif
#ifndef MUON_GEMM_BIG_BK
#define MUON_GEMM_BIG_BK 32
#endif
#ifndef MUON_GEMM_BIG_STAGES
#define MUON_GEMM_BIG_STAGES 4
#endif

namespace muon {

using SmallCfg = GemmCfg<kGemmSmall, kGemmSmall, false>;
using BigCfg = GemmCfg<kGemmBigM, kGemmBigN, MUON_GEMM_BIG_DIRECT != 0, MUON_GEMM_BIG_BK, MUON_GEMM_BIG_STAGES>;

static_assert(kPad % BigCfg::BM == 0 && kPad % BigCfg::BN == 0, "padding must cover the big tile");

template <int MODE, class Cfg, bool SPLIT = false>
__global__ __launch_bounds__(256, (Cfg::kLdsBytes > 80 * 1024) ? 1 : 2) void k_ns_gemm(NsArgs args) {
    __shared__ __attribute__((aligned(16))) unsigned short smem[Cfg::kLdsBytes / 2];
    ns_gemm_tile<MODE, Cfg, SPLIT>(args, smem);
}

// Fixup of the split tiles of a stage, tail or head split (big tiles: 2 x 2 waves of 4 x 4
// blocks of 32 x 32). Each thread takes 4 consecutive accumulator lanes of one wave and
// register index of one split tile, adds the tile's chunks in chunk order and applies the stage's
// epilogue arithmetic, as the tile epilogue does:
//   Gram        A = s2 acc, bf16 at (i, j) and, off the diagonal, at (j, i);
//   polynomial  P = a [i == j < m] + b A + c acc (A read at (j, i)), stored the same way;
//   Apply       X' = s1 acc, bf16 into X'_c at (j, i) and into the row-major X'_r at
//               (i, j) when the next Gram reads it.
// kTailUnitFloats / 1024 blocks per split tile.
template <int MODE>
__global__ __launch_bounds__(256) void k_ns_tail_fix(NsArgs args) {
    using Cfg = BigCfg;
    static_assert(Cfg::NT == 256 && Cfg::TM == 4 && Cfg::TN == 4 && Cfg::WM == 128 && Cfg::WN == 128, "layout");
    constexpr int kBlocksPerTile = kTailUnitFloats / 1024;
    int t = blockIdx.x / kBlocksPerTile;
    const int e = (blockIdx.x % kBlocksPerTile) * 1024 + threadIdx.x * 4;  // accumulator-order index
    int x = 0;
    while (x < 8 && t >= args.xtail[x]) t -= args.xtail[x++];
    if (x >= 8) return;
    const int S = args.xsplit[x];
    int gi, local;
    xcd_slot(args, x, args.xfull[x] + t, gi, local);
    if (gi < 0) return;
    const NsDesc& d = args.d[gi];
    int ti, tj;
    if constexpr (MODE == kModeApply) rect_tile(local, d.m_p / 256, d.tiles, ti, tj);
    else tri_tile(local, d.tiles, ti, tj);
    const float* src = args.tail + (int64_t)(args.xpbase[x] + t * S) * kTailUnitFloats + e;
    floatx4 v = *reinterpret_cast<const floatx4*>(src);
    for (int c = 1; c < S; ++c) {
        const floatx4 p = *reinterpret_cast<const floatx4*>(src + (int64_t)c * kTailUnitFloats);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] += p[q];
    }
    // e = ((wave * 256) + idx) * 64 + lane, idx = (a * 4 + b) * 16 + r
    const int lane0 = e & 63, idx = (e >> 6) & 255, wave = e >> 14;
    const int a = idx >> 6, b = (idx >> 4) & 3, r = idx & 15;
    const int i = ti * 256 + (wave >> 1) * 128 + a * 32 + 8 * (r >> 2) + 4 * (lane0 >> 5) + (r & 3);
    const int64_t ld = d.m_p;
    const float s1 = args.first ? *d.scale : 1.0f;
    const float g2 = s1 * s1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = tj * 256 + (wave & 1) * 128 + b * 32 + ((lane0 + q) & 31);
        float y = v[q];
        if constexpr (MODE == kModeApply) {
            y *= s1;
            const unsigned short h = f2bf(y);
            d.xc_next[kb_off(j, i, ld)] = h;
            if (d.xr_next) d.xr_next[(int64_t)i * d.n_p + j] = h;
        } else {
            unsigned short* dst = (MODE == kModeGram) ? d.a : d.b;
            if constexpr (MODE == kModeGram) {
                y *= g2;
            } else {
                y = fmaf(args.cb, bf2f(d.a[kb_off(j, i, ld)]), args.cc * y);
                if (i == j && i < d.m) y += args.ca;  // P = a I + b A + c A A
            }
            const unsigned short h = f2bf(y);
            dst[kb_off(i, j, ld)] = h;
            if (ti != tj) dst[kb_off(j, i, ld)] = h;
        }
    }
}

template <class Cfg>
static hipError_t launch_cfg(GemmMode mode, const NsArgs& a, hipStream_t s) {
    const dim3 grid(a.total), block(Cfg::NT);
    switch (mode) {
        case kModeGram: hipLaunchKernelGGL((k_ns_gemm<kModeGram, Cfg>), grid, block, 0, s, a); break;
        case kModePoly: hipLaunchKernelGGL((k_ns_gemm<kModePoly, Cfg>), grid, block, 0, s, a); break;
        case kModeApply: hipLaunchKernelGGL((k_ns_gemm<kModeApply, Cfg>), grid, block, 0, s, a); break;
        case kModeFinalO: hipLaunchKernelGGL((k_ns_gemm<kModeFinalO, Cfg>), grid, block, 0, s, a); break;
        case kModeFinalW: hipLaunchKernelGGL((k_ns_gemm<kModeFinalW, Cfg>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_ns_gemm(GemmMode mode, GemmTile tile, const NsArgs& a, hipStream_t s) {
    if (tile != kTileBig) return launch_cfg<SmallCfg>(mode, a, s);
    if (a.tail == nullptr || a.fix_total <= 0) return launch_cfg<BigCfg>(mode, a, s);
    // a stage that splits its tail tiles: the tiles and chunks, then the fixup
    // that adds the chunks and applies the epilogue
    const dim3 grid(a.total), block(BigCfg::NT), fgrid(a.fix_total * (kTailUnitFloats / 1024));
    if (mode == kModeGram) {
        hipLaunchKernelGGL((k_ns_gemm<kModeGram, BigCfg, true>), grid, block, 0, s, a);
        hipLaunchKernelGGL(k_ns_tail_fix<kModeGram>, fgrid, dim3(256), 0, s, a);
    } else if (mode == kModePoly) {
        hipLaunchKernelGGL((k_ns_gemm<kModePoly, BigCfg, true>), grid, block, 0, s, a);
        hipLaunchKernelGGL(k_ns_tail_fix<kModePoly>, fgrid, dim3(256), 0, s, a);
    } else if (mode == kModeApply) {
        hipLaunchKernelGGL((k_ns_gemm<kModeApply, BigCfg, true>), grid, block, 0, s, a);
        hipLaunchKernelGGL(k_ns_tail_fix<kModeApply>, fgrid, dim3(256), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace muon
