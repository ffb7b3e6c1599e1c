// quant_row.hpp -- per-element absmax quantization and workgroup reductions
// shared by the quantize kernels (quant.hip, rmsnorm.hip).
//
// [P1] "2. Absmax Dynamic Activation Quantization" and the
// ActivationQuantizerSTE listing: q = clamp(rne((x * 127) / eta), -128, 127),
// multiply first, then an IEEE division, round half to even.
#pragma once
#include "common.hpp"

namespace bl {

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__device__ inline int8_t quant_one(float x, float eta) {
    float scaled = __fmul_rn(x, kQb);   // x * 127
    float q = __fdiv_rn(scaled, eta);   // ... / eta (IEEE division)
    float r = rintf(q);                 // round half to even
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int8_t)(int)r;
}

__device__ inline uint32_t quant4(float4 v, float eta, int& sum) {
    int8_t a = quant_one(v.x, eta), b = quant_one(v.y, eta), c = quant_one(v.z, eta),
           d = quant_one(v.w, eta);
    sum += (int)a + (int)b + (int)c + (int)d;
    return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
           ((uint32_t)(uint8_t)d << 24);
}

// Block-wide reductions through LDS (one slot per wave).
template <int THREADS>
__device__ inline float block_max(float v, float* red) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < THREADS / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

template <int THREADS>
__device__ inline int block_sum(int v, int* red) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int r = 0;
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) r += red[w];
    return r;
}

}  // namespace bl
