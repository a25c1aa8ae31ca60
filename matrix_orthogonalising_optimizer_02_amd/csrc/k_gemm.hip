// Newton-Schulz GEMM stages on CDNA4 matrix cores ("Muon is Scalable for LLM
// Training", Sec. 2.1 Eq. 2: X <- a X + b (X X^T) X + c (X X^T)^2 X).
//
// Each iteration is three products, all written as C[i][j] = sum_k P[i][k] Q[j][k]
// with both operands K-contiguous in HBM:
//   Gram  A = X X^T   P = Q = X_r ([m_p, n_p])       K = n_p   symmetric output
//   Poly  B = bA+cAA  P = Q = A   ([m_p, m_p])       K = m_p   symmetric (A = A^T)
//   Apply X' = aX+BX  P = B, Q = X_c ([n_p, m_p])    K = m_p   X'_r and X'_c out
// Symmetric outputs compute only the upper-triangular tiles and store each tile
// twice (mirrored). The first iteration folds s = 1 / ||M||_F into the Gram
// (s^2) and Apply (s) epilogues, so X0 never needs its own normalising pass. The
// last Apply writes fp32 O in the input's orientation, or applies Eq. 4 directly.
//
// Tiles: 128 x 128 per 256-thread block (2 x 2 waves of 64 x 64), K step 64,
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation. Operand tiles are staged in LDS
// through registers (double-buffered, one barrier per K step); 16-byte chunks of
// each 128-byte LDS row are XOR-swizzled by (row & 7) so that the per-lane 16-byte
// fragment reads of 32 consecutive rows hit distinct banks.
#include "launch.hpp"

namespace muon {

namespace {

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int WM = BM / 2;  // wave tile rows
constexpr int WN = BN / 2;  // wave tile cols
constexpr int TM = WM / 32; // 32x32 MFMA blocks per wave (rows)
constexpr int TN = WN / 32;
constexpr int LA = BM * BK / 8 / NT;  // 16-byte chunks per thread per operand tile
constexpr int LB = BN * BK / 8 / NT;

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

}  // namespace

template <int MODE>
__global__ __launch_bounds__(NT, 2) void k_ns_gemm(NsArgs args) {
    __shared__ __attribute__((aligned(16))) unsigned short sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) unsigned short sB[2][BN * BK];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int t = xcd_remap(blockIdx.x, args.total);
    int gi = 0;
    while (gi + 1 < args.n && t >= args.d[gi + 1].tile_begin) ++gi;
    const NsDesc& d = args.d[gi];
    int local = t - d.tile_begin;

    constexpr bool kSym = (MODE == kModeGram || MODE == kModePoly);
    int ti, tj;
    if constexpr (kSym) {
        ti = 0;
        while (local >= d.tiles - ti) { local -= d.tiles - ti; ++ti; }
        tj = ti + local;
    } else {
        ti = local / d.tiles;
        tj = local - ti * d.tiles;
    }

    const unsigned short* P;
    const unsigned short* Q;
    int64_t ld;
    int K;
    if constexpr (MODE == kModeGram) { P = d.xr; Q = d.xr; ld = d.n_p; K = d.n_p; }
    else if constexpr (MODE == kModePoly) { P = d.a; Q = d.a; ld = d.m_p; K = d.m_p; }
    else { P = d.b; Q = d.xc; ld = d.m_p; K = d.m_p; }
    const unsigned short* Pt = P + (int64_t)ti * BM * ld;
    const unsigned short* Qt = Q + (int64_t)tj * BN * ld;

    u32x4 ra[LA], rb[LB];
    floatx16 acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // global -> registers for K step 0, registers -> LDS buffer 0
#pragma unroll
    for (int p = 0; p < LA; ++p) {
        const int c = p * NT + tid, row = c >> 3, ch = c & 7;
        ra[p] = *reinterpret_cast<const u32x4*>(Pt + row * ld + ch * 8);
    }
#pragma unroll
    for (int p = 0; p < LB; ++p) {
        const int c = p * NT + tid, row = c >> 3, ch = c & 7;
        rb[p] = *reinterpret_cast<const u32x4*>(Qt + row * ld + ch * 8);
    }
#pragma unroll
    for (int p = 0; p < LA; ++p) {
        const int c = p * NT + tid, row = c >> 3, ch = c & 7;
        *reinterpret_cast<u32x4*>(&sA[0][swz(row, ch)]) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < LB; ++p) {
        const int c = p * NT + tid, row = c >> 3, ch = c & 7;
        *reinterpret_cast<u32x4*>(&sB[0][swz(row, ch)]) = rb[p];
    }
    __syncthreads();

    const int nk = K / BK;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            const int k0 = (kt + 1) * BK;
#pragma unroll
            for (int p = 0; p < LA; ++p) {
                const int c = p * NT + tid, row = c >> 3, ch = c & 7;
                ra[p] = *reinterpret_cast<const u32x4*>(Pt + row * ld + k0 + ch * 8);
            }
#pragma unroll
            for (int p = 0; p < LB; ++p) {
                const int c = p * NT + tid, row = c >> 3, ch = c & 7;
                rb[p] = *reinterpret_cast<const u32x4*>(Qt + row * ld + k0 + ch * 8);
            }
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 af[TM], bfr[TN];
            const int ch = kk * 2 + (lane >> 5);
#pragma unroll
            for (int a = 0; a < TM; ++a) {
                const int row = wm * WM + a * 32 + (lane & 31);
                af[a] = *reinterpret_cast<const bf16x8*>(&sA[cur][swz(row, ch)]);
            }
#pragma unroll
            for (int b = 0; b < TN; ++b) {
                const int row = wn * WN + b * 32 + (lane & 31);
                bfr[b] = *reinterpret_cast<const bf16x8*>(&sB[cur][swz(row, ch)]);
            }
#pragma unroll
            for (int a = 0; a < TM; ++a)
#pragma unroll
                for (int b = 0; b < TN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
        if (more) {
            const int nb = cur ^ 1;
#pragma unroll
            for (int p = 0; p < LA; ++p) {
                const int c = p * NT + tid, row = c >> 3, ch = c & 7;
                *reinterpret_cast<u32x4*>(&sA[nb][swz(row, ch)]) = ra[p];
            }
#pragma unroll
            for (int p = 0; p < LB; ++p) {
                const int c = p * NT + tid, row = c >> 3, ch = c & 7;
                *reinterpret_cast<u32x4*>(&sB[nb][swz(row, ch)]) = rb[p];
            }
        }
        __syncthreads();
    }

    // ---- epilogue. Accumulator element r of a 32x32 block sits at
    // row 8*(r/4) + 4*(lane/32) + r%4, column lane%32.
    const float first_s = args.first ? *d.scale : 1.0f;
    const int row_base = ti * BM + wm * WM;
    const int col_base = tj * BN + wn * WN;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
            const int j = col_base + b * 32 + (lane & 31);
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) {
                const int i0 = row_base + a * 32 + rg * 8 + (lane >> 5) * 4;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[a][b][rg * 4 + e];
                if constexpr (MODE == kModeGram || MODE == kModePoly) {
                    unsigned short* C = (MODE == kModeGram) ? d.a : d.b;
                    const int64_t ldc = d.m_p;
                    unsigned short h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float x;
                        if constexpr (MODE == kModeGram) {
                            x = v[e] * (first_s * first_s);
                        } else {
                            x = fmaf(args.cb, bf2f(d.a[(int64_t)(i0 + e) * ldc + j]), args.cc * v[e]);
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
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = bf2f(d.xr[(int64_t)(i0 + e) * d.n_p + j]);
                        v[e] = fmaf(args.ca, x, v[e]) * first_s;
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
                        // O (or the Eq. 4 update of W) in the input orientation
                        if (!d.tall) {
                            if (j < d.n) {
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int i = i0 + e;
                                    if (i < d.m) {
                                        float* p = d.out + (int64_t)i * d.n + j;
                                        if constexpr (MODE == kModeFinalO) *p = v[e];
                                        else *p = fmaf(-d.upd_coef, v[e], *p * args.decay);
                                    }
                                }
                            }
                        } else if (j < d.n) {
                            float* rowp = d.out + (int64_t)j * d.m;
                            if (((d.m & 3) == 0) && i0 + 3 < d.m) {
                                float4* p = reinterpret_cast<float4*>(rowp + i0);
                                if constexpr (MODE == kModeFinalO) {
                                    *p = make_float4(v[0], v[1], v[2], v[3]);
                                } else {
                                    float4 w = *p;
                                    w.x = fmaf(-d.upd_coef, v[0], w.x * args.decay);
                                    w.y = fmaf(-d.upd_coef, v[1], w.y * args.decay);
                                    w.z = fmaf(-d.upd_coef, v[2], w.z * args.decay);
                                    w.w = fmaf(-d.upd_coef, v[3], w.w * args.decay);
                                    *p = w;
                                }
                            } else {
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    const int i = i0 + e;
                                    if (i < d.m) {
                                        if constexpr (MODE == kModeFinalO) rowp[i] = v[e];
                                        else rowp[i] = fmaf(-d.upd_coef, v[e], rowp[i] * args.decay);
                                    }
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

hipError_t launch_ns_gemm(GemmMode mode, const NsArgs& a, hipStream_t s) {
    const dim3 grid(a.total), block(NT);
    switch (mode) {
        case kModeGram: hipLaunchKernelGGL(k_ns_gemm<kModeGram>, grid, block, 0, s, a); break;
        case kModePoly: hipLaunchKernelGGL(k_ns_gemm<kModePoly>, grid, block, 0, s, a); break;
        case kModeApply: hipLaunchKernelGGL(k_ns_gemm<kModeApply>, grid, block, 0, s, a); break;
        case kModeFinalO: hipLaunchKernelGGL(k_ns_gemm<kModeFinalO>, grid, block, 0, s, a); break;
        case kModeFinalW: hipLaunchKernelGGL(k_ns_gemm<kModeFinalW>, grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace muon
