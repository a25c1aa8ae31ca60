// Launchers for the Newton-Schulz GEMM stages (kernel body in gemm_kernel.hpp).
//
// Two tile configurations are compiled:
//   small: 128 x 128 block tile, register-staged loads, 64 KiB LDS, 2 blocks per CU;
//   big:   256 x 256 block tile (each wave 128 x 128: half the LDS reads per MFMA of
//          the small tile), K step 32 in a 4-deep ring of LDS stages filled by
//          global_load_lds (three K steps of loads in flight), 128 KiB LDS, 1 block per CU.
// The host picks, per stage, the big tile when the launch has enough big tiles to
// fill the GPU, and the small one otherwise (small Gram matrices, small sets).
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

template <int MODE, class Cfg>
__global__ __launch_bounds__(256, (Cfg::kLdsBytes > 80 * 1024) ? 1 : 2) void k_ns_gemm(NsArgs args) {
    __shared__ __attribute__((aligned(16))) unsigned short smem[Cfg::kLdsBytes / 2];
    ns_gemm_tile<MODE, Cfg>(args, smem);
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
    return tile == kTileBig ? launch_cfg<BigCfg>(mode, a, s) : launch_cfg<SmallCfg>(mode, a, s);
}

}  // namespace muon
