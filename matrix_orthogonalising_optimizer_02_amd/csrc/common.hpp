// Shared device helpers and launch descriptors for the gfx950 Muon kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muon {

// Maximum matrices per grouped launch: descriptors travel in the kernel-argument
// segment, so a launch needs no host-to-device copy.
constexpr int kMaxGroup = 16;
// Working dimensions are padded to this multiple (zeros), so every NS5 GEMM tile
// and K step is full and the GEMMs need no bounds checks.
constexpr int kPad = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned short f2bf(float x) {
    __bf16 b = (__bf16)x;  // IEEE round-to-nearest-even
    return __builtin_bit_cast(unsigned short, b);
}

__device__ __forceinline__ float bf2f(unsigned short u) {
    return __uint_as_float(((unsigned)u) << 16);
}

__device__ __forceinline__ unsigned pack2(unsigned short lo, unsigned short hi) {
    return (unsigned)lo | ((unsigned)hi << 16);
}

// Panel-blocked layout of the Newton-Schulz work matrices X_c, A and B: element (r, c)
// of a matrix with `cols` columns (rows padded to a multiple of 256, columns to 32)
// lives in block (r / 256, c / 32), each block 256 x 32 row-major (16 KiB), blocks of a
// 256-row panel consecutive. A GEMM K step over such a matrix reads one contiguous
// block per 256-row operand tile instead of 256 strided 64-byte pieces.
__device__ __forceinline__ int64_t kb_off(int64_t r, int64_t c, int64_t cols) {
    return ((((r >> 8) * (cols >> 5)) + (c >> 5)) << 13) + ((r & 255) << 5) + (c & 31);
}

// Streaming fp32 vector access with the non-temporal hint: the bandwidth-bound passes
// touch each element once, and the hint measurably raises their HBM throughput.
__device__ __forceinline__ floatx4 ld_stream(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
}
__device__ __forceinline__ void st_stream(float* p, floatx4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(p));
}

// max(x, eps) that keeps a NaN x (fmaxf would return eps), so NaN norms propagate.
__device__ __forceinline__ float max_keep_nan(float x, float eps) { return x < eps ? eps : x; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Fixed-order sum over a 256-thread block; every thread gets the result.
__device__ __forceinline__ float block_sum_256(float v, float* red /* >= 4 floats of LDS */) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = ((red[0] + red[1]) + (red[2] + red[3]));
    __syncthreads();
    return s;
}

}  // namespace muon
