// measure.hip -- the ceiling probes declared in include/bitlinear_measure.h:
// an HBM streaming-read kernel and an int8 matrix-core loop, each doing only
// that one thing, so that the forward kernels can be reported as a fraction
// of what this part actually sustains as well as of its published peaks.
#include "bitlinear_measure.h"
#include "kernels.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kSinkWords = 16384;       // 64 KB: one word per workgroup
constexpr int kStreamWavesPerSimd = 4;  // resident wavefronts of the read probe
constexpr int kStreamDepth = 24;        // 16-byte loads in flight per lane (ring)

__device__ inline uint32_t wave_xor(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

// Each wavefront streams one contiguous run of the buffer, the way the
// decode kernels stream their weight rows: 1 KB wave loads (64 lanes x 16
// bytes, non-temporal), kStreamDepth of them in flight as a ring of
// registers, a slot refilled with the block kStreamDepth further on right
// after its use.  The loads go through a buffer descriptor on exactly the
// run (loads past it return zeros without touching memory), so all are
// issued unconditionally and the compiler waits for one block at a time.
// Of the patterns tried on this part this one reads fastest (a ring of 24
// at four wavefronts per SIMD: 7.05 TB/s; rings of 8 or 16, eight waves per
// SIMD, or batches of 16 loads consumed together: 6.95 - 7.05).  Runs are
// whole 1 KB rows of chunks except the last.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, uint64_t n16,
                                                          uint32_t* __restrict__ sink) {
    const uint64_t waves = (uint64_t)gridDim.x * 4;
    const uint64_t w = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint64_t per = ((n16 + waves - 1) / waves + 63) & ~uint64_t(63);   // chunks per wavefront
    const uint64_t begin = w * per;
    const uint64_t end = begin + per < n16 ? begin + per : n16;
    const int nblk = __builtin_amdgcn_readfirstlane((int)(end > begin ? (end - begin) / 64 : 0));
    const uint8_t* run = uniform_ptr(reinterpret_cast<const uint8_t*>(p + (begin < n16 ? begin : 0)));
    const __amdgpu_buffer_rsrc_t res =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(run), 0, nblk * 1024, kBufferRsrcWord3);
    auto ld = [&](int j) { return __builtin_amdgcn_raw_buffer_load_b128(res, lane * 16 + j * 1024, 0, kLoadNonTemporal); };
    nv_u32x4 v[kStreamDepth];
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kStreamDepth; ++i) v[i] = ld(i);
    const int rounds = (nblk + kStreamDepth - 1) / kStreamDepth;
    for (int r = 0; r + 1 < rounds; ++r) {
#pragma unroll
        for (int i = 0; i < kStreamDepth; ++i) {
            x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
            v[i] = ld((r + 1) * kStreamDepth + i);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int i = 0; i < kStreamDepth; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;   // zeros past the run
    for (uint64_t j = begin + (uint64_t)nblk * 64 + lane; j < end; j += 64) {
        const uint4 a = ldnt_u4(p + j);
        x ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    __shared__ uint32_t part[4];
    x = wave_xor(x);
    if (lane == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(const int8_t* __restrict__ xq,
                                                           const uint8_t* __restrict__ packed, int iters,
                                                           int32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    v4i a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = *reinterpret_cast<const v4i*>(xq + (j * 64 + lane) * 16);
        const uint32_t w = *reinterpret_cast<const uint32_t*>(packed + (j * 64 + lane) * 4);
        b[j] = v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                   (int)((w >> 6) & 0x03030303u)};
    }
    v16i acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[t][e] = 0;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j & 3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[j], acc[j & 3], 0, 0, 0);
    }
    uint32_t s = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += (uint32_t)acc[t][e];
    __shared__ uint32_t part[4];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += (uint32_t)__shfl_xor((int)s, off, 64);
    if (lane == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = (int32_t)(part[0] + part[1] + part[2] + part[3]);
}

static int current_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

static int stream_blocks() {
    const int b = current_cus() * kStreamWavesPerSimd;   // 4 SIMDs per CU, 4 waves per workgroup
    return b < kSinkWords ? b : kSinkWords;
}

static int mfma_blocks() {
    const int b = 2 * current_cus();
    return b < kSinkWords ? b : kSinkWords;
}

}  // namespace bl

using namespace bl;

extern "C" {

size_t bitlinear_measure_sink_bytes(void) { return (size_t)kSinkWords * sizeof(uint32_t); }

int bitlinear_measure_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0) return BITLINEAR_EINVAL;
    if (reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return BITLINEAR_EINVAL;
    (void)hipGetLastError();
    hipLaunchKernelGGL(stream_read_kernel, dim3(stream_blocks()), dim3(256), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(buf), (uint64_t)(bytes / 16), sink);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int bitlinear_measure_mfma_i8(const int8_t* xq, const uint8_t* packed, int32_t iters, int32_t* sink,
                              void* stream) {
    if (!xq || !packed || !sink || iters < 1 || iters > (1 << 24)) return BITLINEAR_EINVAL;
    if (reinterpret_cast<uintptr_t>(xq) % 16 != 0 || reinterpret_cast<uintptr_t>(packed) % 4 != 0 ||
        reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return BITLINEAR_EINVAL;
    (void)hipGetLastError();
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(mfma_blocks()), dim3(256), 0, (hipStream_t)stream, xq, packed,
                       (int)iters, sink);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

double bitlinear_measure_mfma_ops(int32_t iters) {
    if (iters < 1 || iters > (1 << 24)) return 0.0;
    // workgroups x 4 wavefronts x iters x 8 MFMAs x (32 * 32 * 32 multiply-adds = 65536 ops)
    return (double)mfma_blocks() * 4.0 * (double)iters * 8.0 * 65536.0;
}

}  // extern "C"
