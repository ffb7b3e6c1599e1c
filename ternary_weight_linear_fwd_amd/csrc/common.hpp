// common.hpp -- definitions shared by the gfx950 kernels of the BitLinear
// library (layout arithmetic, launch helpers, the fused dequant step).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

// Activation quantizer constants ([P1] "2. Absmax Dynamic Activation
// Quantization": Q_b = 127; its listing clamps the scale at 1e-5).
constexpr float kQb = 127.0f;
constexpr float kScaleFloor = 1e-5f;

// Device layout: 64-row groups x 64-k blocks of 1024 bytes (16 per row).
constexpr int kRowsPerGroup = 64;
constexpr int kBlockK = 64;
constexpr int kBlockBytes = 1024;
constexpr int kRowChunkBytes = 16;

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Pointers into the constant address space: loads through them are taken as
// invariant for the kernel's lifetime, so wave-uniform ones become scalar
// loads into SGPRs.
#define BL_CONST __attribute__((address_space(4)))
typedef int nv_i32x4 __attribute__((ext_vector_type(4)));
typedef const BL_CONST nv_i32x4* cint4_ptr;
typedef const BL_CONST int* cint_ptr;
typedef const BL_CONST float* cfloat_ptr;

template <typename T>
__device__ inline const BL_CONST T* as_const(const T* p) {
    return (const BL_CONST T*)(p);
}

// Streaming (non-temporal) 16-byte loads: the data is read once.
typedef unsigned int nv_u32x4 __attribute__((ext_vector_type(4)));
typedef float nv_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ldnt_u4(const void* p) {
    const nv_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nv_u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 ldnt_f4(const void* p) {
    const nv_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nv_f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

// The same loads through pointers the compiler knows to be global, for
// pointers it cannot trace to a kernel argument (read from a descriptor in
// memory): a generic (flat) load also counts against the LDS counter, so
// every LDS access after it would wait for it.
typedef const __attribute__((address_space(1))) nv_u32x4 gnv_u32x4;
typedef const __attribute__((address_space(1))) nv_f32x4 gnv_f32x4;

// Buffer descriptor word 3 of a raw (untyped, 32-bit element) buffer, and
// cache-policy bits of buffer accesses: a store written through the L2 at
// device scope (sc1), a non-temporal load (nt).
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kStoreDeviceScope = 16;
constexpr int kLoadNonTemporal = 2;

// A pointer that is the same in every lane of the wavefront, moved to scalar
// registers (only for values that are wave-uniform by construction).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint4 ldgnt_u4(const void* p) {
    const nv_u32x4 v = __builtin_nontemporal_load((gnv_u32x4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float4 ldg_f4(const void* p) {
    const nv_f32x4 v = *(gnv_f32x4*)p;
    return make_float4(v.x, v.y, v.z, v.w);
}

// Dequantization scale of one token row: s = (eta * gamma) / 127, two float32
// roundings in that order ([P1] BitLinear158.forward step 5; [P5]
// bitlinear_forward listing).
__device__ inline float dequant_scale(float eta, float gamma) {
    float eg = __fmul_rn(eta, gamma);
    return __fdiv_rn(eg, kQb);
}

__device__ inline float dequant(int32_t acc, float s) { return __fmul_rn((float)acc, s); }

// Map three 2-bit codes per byte (values 0, 1, 2 in each byte) to signed
// ternary bytes (-1, 0, +1) with one byte permute: selector byte c picks byte
// c of 0x000100FF, i.e. 0xFF, 0x00, 0x01.
__device__ inline uint32_t codes_to_ternary(uint32_t codes) {
    return __builtin_amdgcn_perm(0u, 0x000100FFu, codes);
}

}  // namespace bl

namespace bl {
// Records the failing HIP call for bitlinear_last_error() (per host thread).
void set_hip_error(hipError_t e, const char* where);
}  // namespace bl

#define BL_HIP_CHECK(expr)                                   \
    do {                                                     \
        hipError_t _e = (expr);                              \
        if (_e != hipSuccess) {                              \
            bl::set_hip_error(_e, #expr);                    \
            return BITLINEAR_EHIP;                           \
        }                                                    \
    } while (0)

// After a kernel launch: the launch's own status (the error state is cleared
// at every API entry, so an earlier failure elsewhere cannot leak in here).
#define BL_LAUNCH_CHECK()                                    \
    do {                                                     \
        hipError_t _e = hipGetLastError();                   \
        if (_e != hipSuccess) {                              \
            bl::set_hip_error(_e, __func__);                 \
            return BITLINEAR_EHIP;                           \
        }                                                    \
    } while (0)
