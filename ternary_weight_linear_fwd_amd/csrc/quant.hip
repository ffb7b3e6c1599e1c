// quant.hip -- per-token absmax INT8 activation quantization on gfx950.
//
// [P1] "2. Absmax Dynamic Activation Quantization" and the
// ActivationQuantizerSTE listing; [P4] "Activation Quantization: 8-Bit Absmax
// Scaling"; [P2] "2. Absmax Activation Quantization" (per token).
//
// One workgroup per token row.  Pass 1 reduces max |x| with wavefront
// butterflies (DPP/permute) and one LDS exchange across the workgroup's
// waves; pass 2 quantizes with one IEEE multiply, one correctly rounded
// division and round-half-even per element and stores four int8 per dword.
// The first R float4 chunks per thread stay in registers between the
// passes (read once from HBM); chunks beyond are read a second time (from
// L2/MALL).  NT: non-temporal loads for the cached chunks.
#include "kernels.hpp"
#include "quant_row.hpp"

namespace bl {

// Store of four quantized values: non-temporal (NTS) or plain.
template <bool NTS>
__device__ __forceinline__ void store_q4(uint32_t* q4, uint32_t v) {
    if constexpr (NTS) __builtin_nontemporal_store(v, q4);
    else *q4 = v;
}

// Quantize one row of K floats (K % 4 == 0, 16-byte aligned).
template <int THREADS, int R, bool NT = true, bool NTS = false>
__device__ inline void quant_row(const float* __restrict__ x, int K, int8_t* __restrict__ xq,
                                 float* __restrict__ eta_out, int32_t* __restrict__ xsum_out) {
    __shared__ float redf[THREADS / 64];
    __shared__ int redi[THREADS / 64];
    const float4* x4 = reinterpret_cast<const float4*>(x);
    uint32_t* q4 = reinterpret_cast<uint32_t*>(xq);
    const int n4 = K >> 2;
    const int t = threadIdx.x;

    float amax = 0.0f;
    float4 cache[R > 0 ? R : 1];
    if constexpr (R > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = t + r * THREADS;
            cache[r] = i < n4 ? (NT ? ldnt_f4(&x4[i]) : x4[i]) : make_float4(0, 0, 0, 0);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(cache[r].x), fabsf(cache[r].y)),
                                     fmaxf(fabsf(cache[r].z), fabsf(cache[r].w))));
        }
    }
    for (int i = t + R * THREADS; i < n4; i += THREADS) {
        float4 v = x4[i];
        amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    amax = block_max<THREADS>(amax, redf);
    const float eta = amax < kScaleFloor ? kScaleFloor : amax;
    const float rcp = quant_recip(eta);

    int sum = 0;
    if constexpr (R > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = t + r * THREADS;
            if (i < n4) store_q4<NTS>(q4 + i, quant4(cache[r], eta, rcp, sum));
        }
    }
    for (int i = t + R * THREADS; i < n4; i += THREADS) store_q4<NTS>(q4 + i, quant4(x4[i], eta, rcp, sum));
    if (t == 0) eta_out[0] = eta;
    if (xsum_out) {
        sum = block_sum<THREADS>(sum, redi);
        if (t == 0) xsum_out[0] = sum;
    }
}

template <int THREADS, int R>
__global__ __launch_bounds__(THREADS) void quant_rows_kernel(const float* __restrict__ x, int K,
                                                             int8_t* __restrict__ xq,
                                                             float* __restrict__ eta,
                                                             int32_t* __restrict__ xsum) {
    const int64_t m = blockIdx.x;
    // Plain loads: 4 - 7% faster than non-temporal ones on 2048-row
    // activations with K = 3200 .. 11008 (as for the grouped kernel);
    // non-temporal stores of x~: 3 - 8% faster than plain ones there
    // (K = 8640 / 3200: 16.6 -> 16.2 us, 6.8 -> 6.2 us).
    quant_row<THREADS, R, false, true>(x + m * K, K, xq + m * K, eta + m, xsum ? xsum + m : nullptr);
}

// Grouped: one workgroup per row descriptor; rows of up to 32768 floats stay
// in registers (512 threads x 16 chunks), longer ones are read twice.  Plain
// loads measured faster than non-temporal ones over the decode step.  NTS:
// non-temporal stores of x~, for contraction kernels that stage x~ through
// LDS (the 70B-shaped sweep at 16 tokens: 3.125 -> 3.074 ms per step); the
// dot4 GEMV reads x~ through the scalar cache and is 0.3% faster after plain
// stores.
constexpr int kGroupedQuantThreads = 512;
template <bool NTS>
__global__ __launch_bounds__(kGroupedQuantThreads) void quant_rows_grouped_kernel(const QuantRow* __restrict__ rows) {
    const QuantRow r = rows[blockIdx.x];
    quant_row<kGroupedQuantThreads, 16, false, NTS>(r.x, r.K, r.xq, r.eta, nullptr);
}

int launch_quantize(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta, int32_t* xsum,
                    hipStream_t stream) {
    if (M == 0) return BITLINEAR_OK;
    const int n4 = (int)(K / 4);
    dim3 grid((unsigned)M);
#define BL_QL(T, R) hipLaunchKernelGGL((quant_rows_kernel<T, R>), grid, dim3(T), 0, stream, x, (int)K, xq, eta, xsum)
    if (n4 <= 256) BL_QL(256, 1);
    else if (n4 <= 512) BL_QL(256, 2);
    else if (n4 <= 1024) BL_QL(256, 4);
    else if (n4 <= 2048) BL_QL(256, 8);
    else if (n4 <= 4096) BL_QL(512, 8);
    else if (n4 <= 8192) BL_QL(1024, 8);
    else BL_QL(1024, 0);
#undef BL_QL
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_quantize_grouped(const QuantRow* rows, int64_t nrows, bool nontemporal, hipStream_t stream) {
    if (nrows == 0) return BITLINEAR_OK;
    if (nontemporal)
        hipLaunchKernelGGL(quant_rows_grouped_kernel<true>, dim3((unsigned)nrows), dim3(kGroupedQuantThreads), 0,
                           stream, rows);
    else
        hipLaunchKernelGGL(quant_rows_grouped_kernel<false>, dim3((unsigned)nrows), dim3(kGroupedQuantThreads), 0,
                           stream, rows);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

}  // namespace bl
