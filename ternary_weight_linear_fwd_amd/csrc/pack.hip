// pack.hip -- absmean ternary weight quantization and 2-bit packing on gfx950.
//
// gamma ([P1] "1. Absmean Weight Quantization", WeightQuantizerSTE listing;
// [P2] "1. Absmean Weight Quantization") is the mean of |W| over the whole
// matrix.  It is computed exactly, independent of summation order: every
// float32 magnitude is sig * 2^(t-149) with sig < 2^24 and 0 <= t <= 253, so
// the kernels add the integer significands into 64-bit bins indexed by t
// (workgroup-private LDS bins, then one global atomic per non-empty bin).  A
// one-thread kernel rebuilds the exact sum, divides it by N*K with base-2^16
// long division and rounds the quotient once to float32 (ties to even).
//
// Ternarization ([P1] "1. Absmean Weight Quantization": Clip(Round(W/gamma),
// -1, 1)) and packing ([P1] "Production Deployment Standards for Edge Systems
// Engineers" item 1; [P5] "Kernel Implementation: The Lookup Table Approach":
// -1 -> 00, 0 -> 01, +1 -> 10) write the device layout documented in
// bitlinear.h, one thread per 32-bit word (16 weights of one row).
#include "kernels.hpp"
#include "ternary.hpp"
#include "pack.hpp"

namespace bl {

size_t gamma_ws_bytes() { return kGammaBins * sizeof(unsigned long long) + 256; }

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* p, size_t n16) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0, 0, 0, 0);
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
    // bytes must be a multiple of 16 and p 16-byte aligned
    const size_t n16 = bytes / 16;
    if (n16 == 0) return BITLINEAR_OK;
    const unsigned blocks = (unsigned)((n16 + 255) / 256 < 4096 ? (n16 + 255) / 256 : 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, stream, (uint4*)p, n16);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

__device__ inline void bin_add(unsigned long long* lbins, float w) {
    const uint32_t bits = __float_as_uint(w) & 0x7fffffffu;
    const uint32_t e = bits >> 23;
    const uint32_t sig = e ? ((bits & 0x7fffffu) | 0x800000u) : (bits & 0x7fffffu);
    const uint32_t t = e ? e - 1 : 0;
    if (sig) atomicAdd(&lbins[t], (unsigned long long)sig);
}

__global__ __launch_bounds__(256) void gamma_bins_kernel(const float4* __restrict__ W, size_t n4,
                                                         unsigned long long* __restrict__ bins) {
    __shared__ unsigned long long lbins[kGammaBins];
    for (int i = threadIdx.x; i < kGammaBins; i += 256) lbins[i] = 0;
    __syncthreads();
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const float4 v = ldnt_f4(&W[i]);
        bin_add(lbins, v.x);
        bin_add(lbins, v.y);
        bin_add(lbins, v.z);
        bin_add(lbins, v.w);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kGammaBins; i += 256)
        if (lbins[i]) atomicAdd(&bins[i], lbins[i]);
}

// Exact mean of |W| from the bins, rounded once to float32, clamped at 1e-5.
__global__ void gamma_final_kernel(const unsigned long long* __restrict__ bins, uint64_t D,
                                   float* __restrict__ gamma, float* __restrict__ gamma_out) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    // The sum in 2^-149 units, as 32-bit limbs with 64-bit headroom: each bin
    // value (< 2^64) shifted by t spreads over three limbs.
    constexpr int NL = 12;  // 384 bits > 318 needed
    uint64_t acc[NL];
    for (int i = 0; i < NL; ++i) acc[i] = 0;
    for (int t = 0; t < 254; ++t) {
        const uint64_t v = bins[t];
        if (!v) continue;
        const int L = t >> 5, b = t & 31;
        const uint64_t lo = (v & 0xffffffffull) << b;  // < 2^63
        const uint64_t hi = (v >> 32) << b;            // < 2^63
        acc[L] += lo & 0xffffffffull;
        acc[L + 1] += (lo >> 32) + (hi & 0xffffffffull);
        acc[L + 2] += hi >> 32;
    }
    for (int i = 0; i + 1 < NL; ++i) {
        acc[i + 1] += acc[i] >> 32;
        acc[i] &= 0xffffffffull;
    }
    // Base-2^16 long division of the sum by D (< 2^40): the remainder stays
    // below D, so (rem << 16) | digit fits in 64 bits.
    constexpr int ND = NL * 2;
    uint32_t q[ND];
    uint64_t rem = 0;
    for (int i = ND - 1; i >= 0; --i) {
        const uint64_t digit = (acc[i >> 1] >> ((i & 1) * 16)) & 0xffffull;
        const uint64_t cur = (rem << 16) | digit;
        q[i] = (uint32_t)(cur / D);
        rem = cur - (uint64_t)q[i] * D;
    }
    // Leading bit P of the integer quotient.
    int P = -1;
    for (int i = ND - 1; i >= 0 && P < 0; --i)
        if (q[i]) P = i * 16 + (31 - __builtin_clz(q[i]));
    float g = 0.0f;
    if (P >= 26) {  // means below 2^-123 end under the clamp anyway
        auto bit = [&](int pos) -> uint32_t { return (q[pos >> 4] >> (pos & 15)) & 1u; };
        uint32_t sig = 0;
        for (int pos = P; pos > P - 24; --pos) sig = (sig << 1) | bit(pos);
        const uint32_t rb = bit(P - 24);
        bool sticky = rem != 0;
        for (int pos = P - 25; pos >= 0 && !sticky; --pos) sticky = bit(pos) != 0;
        int e = P - 149;  // value in [2^e, 2^(e+1))
        if (rb && (sticky || (sig & 1u))) {
            ++sig;
            if (sig == (1u << 24)) { sig >>= 1; ++e; }
        }
        g = __uint_as_float(((uint32_t)(e + 127) << 23) | (sig & 0x7fffffu));
    }
    g = g < kScaleFloor ? kScaleFloor : g;
    gamma[0] = g;
    if (gamma_out) gamma_out[0] = g;
}


// Place the 16 codes of one word: k_local = 4j + i goes to bits 8i + 2j.
__device__ inline uint32_t place16(const uint32_t c[16]) {
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) word |= c[q] << (8 * (q & 3) + 2 * (q >> 2));
    return word;
}

struct WordPos {
    int64_t n, k0;
};

__device__ inline WordPos word_pos(int64_t i, int64_t Kb) {
    const int64_t d = i & 3, r = (i >> 2) & 63, gb = i >> 8;
    const int64_t g = gb / Kb, b = gb - g * Kb;
    return {g * 64 + r, b * 64 + d * 16};
}

__global__ __launch_bounds__(256) void ternarize_pack_kernel(const float* __restrict__ W, int64_t N,
                                                             int64_t K, int64_t Kb,
                                                             const float* __restrict__ gamma_p,
                                                             uint32_t* __restrict__ packed,
                                                             int64_t nwords) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nwords) return;
    const WordPos p = word_pos(i, Kb);
    uint32_t word = 0x55555555u;  // all zero weights (pad rows and columns)
    if (p.n < N && p.k0 < K) {
        const float gamma = gamma_p[0];
        const float4* src = reinterpret_cast<const float4*>(W + p.n * K + p.k0);
        uint32_t c[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 f = ldnt_f4(&src[v]);
            c[4 * v + 0] = ternary_code(f.x, gamma);
            c[4 * v + 1] = ternary_code(f.y, gamma);
            c[4 * v + 2] = ternary_code(f.z, gamma);
            c[4 * v + 3] = ternary_code(f.w, gamma);
        }
        word = place16(c);
    }
    packed[i] = word;
}

__global__ __launch_bounds__(256) void pack_ternary_kernel(const int8_t* __restrict__ Wt, int64_t N,
                                                           int64_t K, int64_t Kb,
                                                           uint32_t* __restrict__ packed,
                                                           int64_t nwords, int32_t* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nwords) return;
    const WordPos p = word_pos(i, Kb);
    uint32_t word = 0x55555555u;
    if (p.n < N && p.k0 < K) {
        const uint4 raw = *reinterpret_cast<const uint4*>(Wt + p.n * K + p.k0);
        const uint32_t v[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t c[16];
        int nbad = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int w = (int8_t)((v[q >> 2] >> (8 * (q & 3))) & 0xff);
            const bool ok = w >= -1 && w <= 1;
            nbad += !ok;
            c[q] = ok ? (uint32_t)(w + 1) : 1u;
        }
        word = place16(c);
        if (nbad && bad) atomicAdd(bad, nbad);
    }
    packed[i] = word;
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ packed, int64_t N,
                                                     int64_t K, int64_t Kb, int8_t* __restrict__ Wt,
                                                     int64_t nwords, int32_t* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= nwords) return;
    const WordPos p = word_pos(i, Kb);
    if (p.n >= N || p.k0 >= K) return;
    const uint32_t word = packed[i];
    uint32_t out[4] = {0, 0, 0, 0};
    int nbad = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint32_t code = (word >> (8 * (q & 3) + 2 * (q >> 2))) & 3u;
        nbad += code == 3u;
        const int w = code == 3u ? 0 : (int)code - 1;
        out[q >> 2] |= ((uint32_t)(uint8_t)(int8_t)w) << (8 * (q & 3));
    }
    *reinterpret_cast<uint4*>(Wt + p.n * K + p.k0) = make_uint4(out[0], out[1], out[2], out[3]);
    if (nbad && bad) atomicAdd(bad, nbad);
}

static int64_t layout_words(int64_t N, int64_t K) {
    return ceil_div(N, 64) * ceil_div(K, 64) * 256;
}

int launch_gamma(const float* W, int64_t N, int64_t K, float* gamma_dev, void* ws,
                 hipStream_t stream) {
    unsigned long long* bins = (unsigned long long*)ws;
    float* gamma_ws = (float*)((char*)ws + kGammaBins * sizeof(unsigned long long));
    int rc = launch_fill_zero(bins, kGammaBins * sizeof(unsigned long long), stream);
    if (rc) return rc;
    const size_t n4 = (size_t)(N * K / 4);
    const unsigned blocks = (unsigned)(n4 / 256 + 1 < 2048 ? n4 / 256 + 1 : 2048);
    hipLaunchKernelGGL(gamma_bins_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(W), n4, bins);
    BL_LAUNCH_CHECK();
    hipLaunchKernelGGL(gamma_final_kernel, dim3(1), dim3(64), 0, stream, bins,
                       (uint64_t)N * (uint64_t)K, gamma_ws, gamma_dev);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma_dev,
                        void* ws, hipStream_t stream) {
    int rc = launch_gamma(W, N, K, gamma_dev, ws, stream);
    if (rc) return rc;
    const float* gamma_ws = (const float*)((const char*)ws + kGammaBins * sizeof(unsigned long long));
    const int64_t nwords = layout_words(N, K);
    hipLaunchKernelGGL(ternarize_pack_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0,
                       stream, W, N, K, ceil_div(K, 64), gamma_ws, (uint32_t*)packed, nwords);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_ternarize_pack(const float* W, int64_t N, int64_t K, const float* gamma_dev,
                          uint8_t* packed, hipStream_t stream) {
    const int64_t nwords = layout_words(N, K);
    hipLaunchKernelGGL(ternarize_pack_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0,
                       stream, W, N, K, ceil_div(K, 64), gamma_dev, (uint32_t*)packed, nwords);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

__global__ void zero_i32_kernel(int32_t* p) { *p = 0; }

int launch_zero_i32(int32_t* p, hipStream_t stream) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, stream, p);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_pack_ternary(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed, int32_t* bad,
                        hipStream_t stream) {
    const int64_t nwords = layout_words(N, K);
    hipLaunchKernelGGL(pack_ternary_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0,
                       stream, Wt, N, K, ceil_div(K, 64), (uint32_t*)packed, nwords, bad);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wt, int32_t* bad,
                  hipStream_t stream) {
    const int64_t nwords = layout_words(N, K);
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)ceil_div(nwords, 256)), dim3(256), 0, stream,
                       (const uint32_t*)packed, N, K, ceil_div(K, 64), Wt, nwords, bad);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

}  // namespace bl
