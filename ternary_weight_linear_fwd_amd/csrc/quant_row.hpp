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

// The reciprocal the fast path of quant4 multiplies by: fl(1 / eta), or NaN
// (no fast path) when it would be subnormal.  One per row.
__device__ inline float quant_recip(float eta) {
    return eta < 0x1p125f ? __fdiv_rn(1.0f, eta) : __builtin_nanf("");
}

// Four elements of quant_one, the same bits with a division only where it
// can matter.  With a = fl(x * 127) and q = a / eta, |q| <= 127 (eta is at
// least every |x| of the row), and p = fl(a * fl(1 / eta)) is within
// |q| (2^-24 + 2^-24 + 2^-48) < 1.6e-5 of q, while fl(q) is within
// |q| 2^-24 < 7.6e-6 of q.  So when p is farther than 2^-12 from every
// half-integer, fl(q) lies strictly between the same two half-integers and
// rint(fl(q)) = rint(p).  Otherwise (a tie or a near tie of fl(q), or a
// non-finite p) the lane takes the IEEE division.
__device__ inline uint32_t quant4(float4 v, float eta, float rcp, int& sum) {
    const float a[4] = {__fmul_rn(v.x, kQb), __fmul_rn(v.y, kQb), __fmul_rn(v.z, kQb), __fmul_rn(v.w, kQb)};
    float n[4];
    bool exact = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float p = __fmul_rn(a[j], rcp);
        n[j] = rintf(p);
        exact |= !(fabsf(p - n[j]) < 0.5f - 0x1p-12f);   // also true for NaN / inf
    }
    if (exact) {
#pragma unroll
        for (int j = 0; j < 4; ++j) n[j] = rintf(__fdiv_rn(a[j], eta));
    }
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int8_t q = (int8_t)(int)fminf(fmaxf(n[j], -128.0f), 127.0f);
        sum += (int)q;
        out |= (uint32_t)(uint8_t)q << (8 * j);
    }
    return out;
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
