// Attainable ceilings of the two rooflines the optimizer step is measured against: a
// streaming fp32 copy (the HBM-bound passes' yardstick) and a register-only bf16 MFMA
// loop (the Newton-Schulz GEMMs' yardstick). Neither is part of the optimizer step;
// the benchmark times them on the same GPU in the same run, beside the spec peaks
// (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16).
#include "../../include/muon_rocm.h"
#include "abi_internal.hpp"
#include "launch.hpp"

#define MUON_API extern "C" __attribute__((visibility("default")))

namespace muon {
namespace {

// Copy: 256 threads, kCopyVec float4 per thread, one contiguous 32 KiB chunk per block,
// every load of a thread issued before its stores, non-temporal hints (the access
// pattern of the streaming passes of the step). Of the variants measured on MI355X
// (2, 4, 8 and 16 float4 per thread; 64 to 1024 threads; plain or non-temporal loads and
// stores; a persistent grid) this one copies fastest, 6.36 TB/s on 1 GiB.
constexpr int kCopyVec = 8;
constexpr int64_t kCopyBlockElems = 256 * 4 * kCopyVec;

__global__ __launch_bounds__(256) void k_ceiling_copy(const float* __restrict__ src, float* __restrict__ dst,
                                                      int64_t n) {
    const int64_t base = (int64_t)blockIdx.x * kCopyBlockElems;
    if (base + kCopyBlockElems <= n) {
        floatx4 v[kCopyVec];
#pragma unroll
        for (int k = 0; k < kCopyVec; ++k) v[k] = ld_stream(src + base + (int64_t)(k * 256 + threadIdx.x) * 4);
#pragma unroll
        for (int k = 0; k < kCopyVec; ++k) st_stream(dst + base + (int64_t)(k * 256 + threadIdx.x) * 4, v[k]);
    } else {
        for (int64_t i = base + threadIdx.x; i < n; i += 256) dst[i] = src[i];
    }
}

// MFMA loop: each wave keeps 16 independent 32 x 32 fp32 accumulators (256 VGPRs, as a
// GEMM wave's 128 x 128 tile does) and issues `iters` rounds of 16
// v_mfma_f32_32x32x16_bf16 on operands held in registers. The matrix cores' power, and
// with it the clock the chip sustains, depends on how many operand bits toggle, so the
// operands change every round as a GEMM's do: each of the eight operand words of a lane
// steps by a constant and is masked to sign, 7 mantissa bits and a fixed exponent (bf16
// values of magnitude in [0.5, 1)). Three VALU operations per word per round sit in the
// shadow of 16 MFMAs. No memory traffic apart from one checksum per wave at the end,
// which keeps the products live.
constexpr int kMfmaAcc = 16;
constexpr unsigned kMfmaStep = 0x00250025u;   // added to both bf16 halves of a word
constexpr unsigned kMfmaMask = 0x807F807Fu;   // sign and mantissa bits kept
constexpr unsigned kMfmaExp = 0x3F003F00u;    // exponent of [0.5, 1)

__device__ __forceinline__ unsigned mfma_word(unsigned w) { return ((w + kMfmaStep) & kMfmaMask) | kMfmaExp; }

__global__ __launch_bounds__(256) void k_ceiling_mfma(float* out, int iters) {
    const unsigned lane = threadIdx.x & 63;
    u32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        a[e] = ((lane * 0x01030107u + e * 0x00110013u) & kMfmaMask) | kMfmaExp;
        b[e] = ((lane * 0x02050309u + e * 0x00170019u) & kMfmaMask) | kMfmaExp;
    }
    floatx16 acc[kMfmaAcc];
#pragma unroll
    for (int t = 0; t < kMfmaAcc; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
        for (int t = 0; t < kMfmaAcc; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[t], 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = mfma_word(a[e]);
            b[e] = mfma_word(b[e]);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < kMfmaAcc; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[t][r];
    s = wave_sum(s);
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace muon

MUON_API int muon_ceiling_copy(const float* src, float* dst, int64_t n, void* stream) {
    using muon::set_last_error;
    set_last_error(MUON_OK, "");
    if (n < 0 || (n > 0 && (!src || !dst))) return set_last_error(MUON_ERR_INVALID_ARG, "n < 0 or NULL pointer");
    if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15)
        return set_last_error(MUON_ERR_ALIGN, "src or dst not 16-byte aligned");
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t bytes = uintptr_t(n) * 4;
    if (n > 0 && s0 < d0 + bytes && d0 < s0 + bytes) return set_last_error(MUON_ERR_ALIAS, "src and dst overlap");
    if (n == 0) return MUON_OK;
    const int64_t blocks = (n + muon::kCopyBlockElems - 1) / muon::kCopyBlockElems;
    if (blocks >= (int64_t(1) << 31)) return set_last_error(MUON_ERR_TOO_LARGE, "copy above 2^31 blocks");
    hipLaunchKernelGGL(muon::k_ceiling_copy, dim3(unsigned(blocks)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), src, dst, n);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MUON_OK : set_last_error(MUON_ERR_HIP, std::string("copy: ") + hipGetErrorString(e));
}

MUON_API int muon_ceiling_mfma(float* out, int32_t blocks, int32_t iters, double* flops, void* stream) {
    using muon::set_last_error;
    set_last_error(MUON_OK, "");
    if (blocks < 0 || iters < 0 || (blocks > 0 && !out))
        return set_last_error(MUON_ERR_INVALID_ARG, "blocks < 0, iters < 0 or NULL out");
    if (reinterpret_cast<uintptr_t>(out) & 3) return set_last_error(MUON_ERR_ALIGN, "out not 4-byte aligned");
    if (flops) *flops = double(blocks) * 4.0 * double(iters) * muon::kMfmaAcc * (32.0 * 32.0 * 16.0 * 2.0);
    if (blocks == 0) return MUON_OK;
    hipLaunchKernelGGL(muon::k_ceiling_mfma, dim3(unsigned(blocks)), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), out, iters);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MUON_OK : set_last_error(MUON_ERR_HIP, std::string("mfma loop: ") + hipGetErrorString(e));
}
