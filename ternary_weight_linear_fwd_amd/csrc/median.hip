// median.hip -- the absmedian weight scale on gfx950.
//
// [P2] "Scaling Laws and Empirical Benchmarks" (BitNet b1.58
// Reloaded: the quantization baseline adjusted to the median, "Absmedian",
// rather than the mean).  gamma = median of |W| over the matrix; for an even
// count the mean of the two middle magnitudes, rounded once to float32;
// clamped below at 1e-5; the ternarization is the absmean one with this scale.
//
// Selection.  Non-negative float32 magnitudes order like their 31-bit
// patterns, so the two middle ranks r0 = (D-1)/2 and r1 = D/2 are found by a
// three-pass radix select on the bits (11 + 10 + 10): each pass histograms the
// magnitudes that match the prefixes chosen so far (workgroup-private LDS
// counters, then 64-bit global atomics) and one thread walks the histogram to
// extend each rank's prefix.  Both ranks share the passes.  The mean of the
// two magnitudes is formed in float64 (exact operands; 53 >= 2 * 24 + 2 bits,
// so rounding the float64 sum to float32 rounds the exact mean correctly).
#include "median.hpp"
#include "pack.hpp"

namespace bl {

struct MedianState {
    unsigned long long rank[2];   // remaining rank inside the current prefix
    uint32_t prefix[2];           // bits chosen so far (pass 1: 11, 2: 21, 3: 31)
    float gamma;
    uint32_t pad;
};

constexpr size_t kHist1 = 2048, kHist2 = 1024;
constexpr size_t kOffH1 = 0;
constexpr size_t kOffH2 = kOffH1 + kHist1 * 8;
constexpr size_t kOffH3 = kOffH2 + 2 * kHist2 * 8;
constexpr size_t kOffState = kOffH3 + 2 * kHist2 * 8;
constexpr size_t kMedianWs = kOffState + 256;

size_t median_ws_bytes() { return kMedianWs; }

// Pass 1: histogram of bits 30..20 of every magnitude.
__global__ __launch_bounds__(256) void median_hist1_kernel(const float4* __restrict__ W, size_t n4,
                                                           unsigned long long* __restrict__ hist) {
    __shared__ uint32_t h[kHist1];
    for (int i = threadIdx.x; i < (int)kHist1; i += 256) h[i] = 0;
    __syncthreads();
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const float4 v = ldnt_f4(&W[i]);
        atomicAdd(&h[(__float_as_uint(v.x) & 0x7fffffffu) >> 20], 1u);
        atomicAdd(&h[(__float_as_uint(v.y) & 0x7fffffffu) >> 20], 1u);
        atomicAdd(&h[(__float_as_uint(v.z) & 0x7fffffffu) >> 20], 1u);
        atomicAdd(&h[(__float_as_uint(v.w) & 0x7fffffffu) >> 20], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < (int)kHist1; i += 256)
        if (h[i]) atomicAdd(&hist[i], (unsigned long long)h[i]);
}

// Passes 2 and 3: for each rank, histogram bits [shift, shift + 10) of the
// magnitudes whose bits above match its prefix.
__device__ inline void hist_match(uint32_t key, int shift, uint32_t p0, uint32_t p1, uint32_t* h0,
                                  uint32_t* h1) {
    const uint32_t top = key >> (shift + 10), bin = (key >> shift) & 1023u;
    if (top == p0) atomicAdd(&h0[bin], 1u);
    if (top == p1) atomicAdd(&h1[bin], 1u);
}

__global__ __launch_bounds__(256) void median_hist_next_kernel(const float4* __restrict__ W, size_t n4,
                                                               int shift,
                                                               const MedianState* __restrict__ st,
                                                               unsigned long long* __restrict__ hist) {
    __shared__ uint32_t h0[kHist2], h1[kHist2];
    for (int i = threadIdx.x; i < (int)kHist2; i += 256) h0[i] = h1[i] = 0;
    __syncthreads();
    const uint32_t p0 = st->prefix[0], p1 = st->prefix[1];
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        const float4 v = ldnt_f4(&W[i]);
        hist_match(__float_as_uint(v.x) & 0x7fffffffu, shift, p0, p1, h0, h1);
        hist_match(__float_as_uint(v.y) & 0x7fffffffu, shift, p0, p1, h0, h1);
        hist_match(__float_as_uint(v.z) & 0x7fffffffu, shift, p0, p1, h0, h1);
        hist_match(__float_as_uint(v.w) & 0x7fffffffu, shift, p0, p1, h0, h1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < (int)kHist2; i += 256) {
        if (h0[i]) atomicAdd(&hist[i], (unsigned long long)h0[i]);
        if (h1[i]) atomicAdd(&hist[kHist2 + i], (unsigned long long)h1[i]);
    }
}

// Walk a histogram: the bin holding `rank`, and the rank left inside it.
__device__ inline uint32_t walk(const unsigned long long* h, int nbins, unsigned long long& rank) {
    unsigned long long below = 0;
    for (int b = 0; b < nbins; ++b) {
        if (rank < below + h[b]) {
            rank -= below;
            return (uint32_t)b;
        }
        below += h[b];
    }
    rank = 0;   // unreachable for a consistent histogram
    return (uint32_t)(nbins - 1);
}

// pass 1 (both ranks from the one histogram), 2 and 3 (one histogram each);
// after pass 3 the prefixes are the two magnitudes and gamma is formed.
__global__ void median_select_kernel(const unsigned long long* __restrict__ hist, int pass,
                                     uint64_t D, MedianState* __restrict__ st,
                                     float* __restrict__ gamma_out) {
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    if (pass == 1) {
        st->rank[0] = (D - 1) / 2;
        st->rank[1] = D / 2;
        for (int t = 0; t < 2; ++t) st->prefix[t] = walk(hist, (int)kHist1, st->rank[t]);
        return;
    }
    for (int t = 0; t < 2; ++t) {
        const uint32_t b = walk(hist + t * kHist2, (int)kHist2, st->rank[t]);
        st->prefix[t] = (st->prefix[t] << 10) | b;
    }
    if (pass == 3) {
        const double a = (double)__uint_as_float(st->prefix[0]);
        const double c = (double)__uint_as_float(st->prefix[1]);
        float g = (float)((a + c) * 0.5);
        if (!(g >= kScaleFloor)) g = kScaleFloor;
        st->gamma = g;
        if (gamma_out) gamma_out[0] = g;
    }
}

int launch_absmedian_gamma(const float* W, int64_t N, int64_t K, float* gamma_dev, void* ws,
                           const float** gamma_ws, hipStream_t stream) {
    char* base = (char*)ws;
    unsigned long long* h1 = (unsigned long long*)(base + kOffH1);
    unsigned long long* h2 = (unsigned long long*)(base + kOffH2);
    unsigned long long* h3 = (unsigned long long*)(base + kOffH3);
    MedianState* st = (MedianState*)(base + kOffState);
    int rc = launch_fill_zero(base, kMedianWs, stream);
    if (rc) return rc;
    const uint64_t D = (uint64_t)N * (uint64_t)K;
    const size_t n4 = (size_t)(D / 4);   // K % 16 == 0
    const unsigned blocks = (unsigned)(n4 / 256 + 1 < 2048 ? n4 / 256 + 1 : 2048);
    const float4* W4 = reinterpret_cast<const float4*>(W);
    hipLaunchKernelGGL(median_hist1_kernel, dim3(blocks), dim3(256), 0, stream, W4, n4, h1);
    BL_LAUNCH_CHECK();
    hipLaunchKernelGGL(median_select_kernel, dim3(1), dim3(64), 0, stream, h1, 1, D, st, nullptr);
    BL_LAUNCH_CHECK();
    hipLaunchKernelGGL(median_hist_next_kernel, dim3(blocks), dim3(256), 0, stream, W4, n4, 10,
                       (const MedianState*)st, h2);
    BL_LAUNCH_CHECK();
    hipLaunchKernelGGL(median_select_kernel, dim3(1), dim3(64), 0, stream, h2, 2, D, st, nullptr);
    BL_LAUNCH_CHECK();
    hipLaunchKernelGGL(median_hist_next_kernel, dim3(blocks), dim3(256), 0, stream, W4, n4, 0,
                       (const MedianState*)st, h3);
    BL_LAUNCH_CHECK();
    hipLaunchKernelGGL(median_select_kernel, dim3(1), dim3(64), 0, stream, h3, 3, D, st, gamma_dev);
    BL_LAUNCH_CHECK();
    *gamma_ws = &st->gamma;
    return BITLINEAR_OK;
}

int launch_pack_weights_absmedian(const float* W, int64_t N, int64_t K, uint8_t* packed,
                                  float* gamma_dev, void* ws, const float** gamma_ws,
                                  hipStream_t stream) {
    int rc = launch_absmedian_gamma(W, N, K, gamma_dev, ws, gamma_ws, stream);
    if (rc) return rc;
    return launch_ternarize_pack(W, N, K, *gamma_ws, packed, stream);
}

}  // namespace bl
