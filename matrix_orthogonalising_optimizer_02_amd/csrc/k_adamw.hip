// AdamW for the parameters that the hybrid optimizer keeps off Muon: biases,
// normalisation weights and everything outside the transformer blocks ("Scaling Muon
// for Diffusion Transformers", setup paragraph; "Muon is Scalable for LLM Training",
// Sec. 2.2, matching-update-RMS paragraph, decoupled decay as in Eq. 3).
//
//   m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g^2
//   W <- (1 - lr wd) W - (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps)
//
// HBM-bound: 28 bytes per element (read W, G, m, v; write W, m, v). One block handles
// 4096 consecutive elements of one tensor as 16 per thread in four float4, all loads
// of the block issued before its stores.
#include "launch.hpp"

namespace muon {

__device__ __forceinline__ float adam_elem(const AdamArgs& a, float w, float g, float& m, float& v) {
    m = fmaf(a.beta1, m, a.one_minus_beta1 * g);
    v = fmaf(a.beta2, v, a.one_minus_beta2 * (g * g));
    const float den = fmaf(sqrtf(v), a.inv_sqrt_bc2, a.eps);
    return fmaf(-a.lr_bc1, m / den, w * a.decay);
}

__global__ __launch_bounds__(256) void k_adamw(AdamArgs args) {
    const int t = blockIdx.x;
    int lo = 0, hi = args.n - 1;  // last tensor whose blk_begin <= t
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (args.d[mid].blk_begin <= t) lo = mid;
        else hi = mid - 1;
    }
    const AdamDesc& d = args.d[lo];
    const int64_t base = (int64_t)(t - d.blk_begin) * kAdamBlockElems;
    constexpr int kV = kAdamBlockElems / 256 / 4;
    if (base + kAdamBlockElems <= d.n) {
        floatx4 wv[kV], gv[kV], mv[kV], vv[kV];
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int64_t i = base + (int64_t)(k * 256 + threadIdx.x) * 4;
            wv[k] = ld_stream(d.w + i);
            gv[k] = ld_stream(d.g + i);
            mv[k] = ld_stream(d.m + i);
            vv[k] = ld_stream(d.v + i);
        }
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int64_t i = base + (int64_t)(k * 256 + threadIdx.x) * 4;
            floatx4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float m = mv[k][e], v = vv[k][e];
                w[e] = adam_elem(args, wv[k][e], gv[k][e], m, v);
                mv[k][e] = m;
                vv[k][e] = v;
            }
            st_stream(d.w + i, w);
            st_stream(d.m + i, mv[k]);
            st_stream(d.v + i, vv[k]);
        }
    } else {
        for (int64_t i = base + threadIdx.x; i < d.n; i += 256) {
            float m = d.m[i], v = d.v[i];
            d.w[i] = adam_elem(args, d.w[i], d.g[i], m, v);
            d.m[i] = m;
            d.v[i] = v;
        }
    }
}

hipError_t launch_adamw(const AdamArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_adamw, dim3(a.total), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace muon
