// rmsnorm.hip -- RMSNorm without affine parameters fused with the per-token
// absmax INT8 quantizer, one read of x.
//
// [P1] pipeline box 1 ("RMSNorm") and step 1 of BitLinear158.forward in
// "Production PyTorch Implementation: BitLinear b1.58 Layer": norm =
// rsqrt(mean(x^2) + 1e-6), x_norm = x * norm, then the absmax quantizer of
// step 2 on x_norm; [P1] "2. Absmax Dynamic Activation Quantization" (the
// normalization has no learnable affine parameters); [P2] "2. Absmax
// Activation Quantization" (normalization precedes quantization).
//
// Float semantics, fixed so that the result is a function of x alone:
//   ms     = the exact mean of the squares, rounded once to float32 (RNE)
//   norm   = 1 / sqrt(ms + 1e-6): an IEEE add, square root and division
//            (the square root corrected to the correctly rounded one)
//   x_norm = x * norm;   eta = max(max_k |x_norm|, 1e-5);   xq as usual.
// Rounding is monotone, so max_k |x_norm| = fl(max_k |x| * norm): eta needs
// only the row's max |x|, and x_norm is formed on the fly while quantizing.
//
// The exact mean, cheaply.  Every float32 square is exact in float64, and a
// float64 sum of K non-negative terms in any order is within (K-1) * 2^-53 of
// the true sum (relative), the division by K adds one more rounding.  Each row
// therefore forms S in float64 with the same butterfly reductions as max |x|;
// when the interval S/K * (1 +- (K+4) 2^-52) holds no float32 rounding
// boundary, the float32 nearest to S/K is the correctly rounded exact mean.
// Otherwise (exact ties, results within ~2^-40 of a boundary, very long rows)
// the row takes an exact path in two tiers.  First every square is summed in
// 128-bit integers of a fixed-point window below the row's largest square
// (window_add): exact for every element within 2^28 of the largest, and the
// rest contribute their whole units while flagging their dropped remainders;
// the quotient by K is then rounded exactly, or -- when remainders were
// dropped -- accepted only if both ends of the interval they span round
// alike.  Rows that stay undecided (remainders that could tip a tie) add every
// square sig^2 * 2^(2t-298) (|x| = sig * 2^(t-149)), split in two 24-bit
// halves, to a per-exponent 64-bit LDS bin; one thread assembles the 640-bit
// sum, divides it by K limb by limb and rounds the quotient.
#include "quant_row.hpp"
#include "rmsnorm.hpp"

namespace bl {

constexpr float kRmsEps = 1e-6f;
constexpr int kBins = 254;   // t = 0 .. 253
constexpr int kLimbs = 21;   // 672 bits >= 2 * 253 + 24 + 55

// Correctly rounded float32 square root.  The device square root may be off
// by one unit; the candidate is moved to the neighbour whose rounding interval
// holds sqrt(t), decided exactly: a midpoint of two adjacent floats has at most
// 25 significant bits, so its square is exact in float64 (no ties can occur).
__device__ inline float sqrt_rn(float t) {
    float s = __fsqrt_rn(t);
    if (!(t > 0.0f) || isinf(t)) return s;
    const double td = (double)t;
    for (int it = 0; it < 2; ++it) {
        const float up = nextafterf(s, INFINITY), dn = nextafterf(s, 0.0f);
        const double mu = 0.5 * ((double)s + (double)up), md = 0.5 * ((double)s + (double)dn);
        if (td > mu * mu) s = up;
        else if (td < md * md) s = dn;
        else break;
    }
    return s;
}

__device__ inline double wave_sum_f64(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// The rounding interval of a non-negative float32 r: the exact values that
// round (to nearest, ties to even) to r lie within [lo, hi]; ties sit on the
// bounds, which the caller treats as ambiguous.
__device__ inline void f32_rounding_interval(float r, double& lo, double& hi) {
    const double over = 0x1p128 - 0x1p103;   // midpoint of FLT_MAX and 2^128
    const double dr = (double)r;
    if (isinf(r)) {
        lo = over;
        hi = INFINITY;
        return;
    }
    lo = r == 0.0f ? -1.0 : 0.5 * (dr + (double)nextafterf(r, 0.0f));
    hi = r == 3.40282347e38f ? over : 0.5 * (dr + (double)nextafterf(r, INFINITY));
}

__device__ inline int big_getbit(const uint32_t* big, int p) { return (big[p >> 5] >> (p & 31)) & 1; }

// Bits [32j, 32j + 32) of v * 2^s, where rel = s - 32j and v < 2^56: the low
// 32 bits of v << rel (bits past 64 do not reach them), or of v >> -rel.
__device__ inline uint64_t limb_piece(uint64_t v, int rel) {
    if (rel >= 32 || rel <= -64) return 0;
    return (rel >= 0 ? v << rel : v >> -rel) & 0xffffffffull;
}

// big = the exact sum over bins (as in exact_mean_f32), limb by limb in
// parallel: lane j of the first wave adds the pieces of every bin value that
// fall into limb j (at most 2 * kBins pieces below 2^32: no overflow of 64
// bits), then one thread propagates the carries.  Called by every thread of
// the workgroup (it synchronizes).
__device__ void exact_limbs(const unsigned long long (*bins)[2], uint32_t* big, unsigned long long* raw, int t) {
    if (t < kLimbs) {
        const int j = t;
        // lo halves sit at 2^(2b), hi halves at 2^(2b + 24); only bins with
        // -64 < shift - 32j < 32 reach limb j.
        const int b0 = 16 * j - 44 > 0 ? 16 * j - 44 : 0;
        const int b1 = 16 * j + 16 < kBins ? 16 * j + 16 : kBins;
        uint64_t acc = 0;
        for (int b = b0; b < b1; ++b) {
            acc += limb_piece(bins[b][1], 2 * b - 32 * j);
            acc += limb_piece(bins[b][0], 2 * b + 24 - 32 * j);
        }
        raw[j] = acc;
    }
    __syncthreads();
    if (t == 0) {
        uint64_t carry = 0;
        for (int j = 0; j < kLimbs; ++j) {
            const uint64_t a = raw[j] + carry;
            big[j] = (uint32_t)a;
            carry = a >> 32;
        }
    }
    __syncthreads();
}

// The float32 nearest to S / K, by exact integer arithmetic (one thread), S
// the sum over bins: bins[t] = {sum of hi halves, sum of lo halves}, the
// squares in bin t adding up to (hi * 2^24 + lo) * 2^(2t - 298).
__device__ float exact_mean_f32(uint32_t* big, uint64_t K) {
    // big holds S, the exact sum over bins (exact_limbs).
    // Q = floor(S / K) limb by limb (rem < K < 2^31), in units of 2^-298.
    uint64_t rem = 0;
    for (int i = kLimbs - 1; i >= 0; --i) {
        const uint64_t cur = (rem << 32) | big[i];
        big[i] = (uint32_t)(cur / K);
        rem = cur % K;
    }
    int L = -1;   // top set bit of Q
    for (int i = kLimbs - 1; i >= 0 && L < 0; --i)
        if (big[i]) L = 32 * i + 31 - __builtin_clz(big[i]);
    if (L < 0) return 0.0f;                       // S / K < 2^-298
    const int a_lead = L - 298;                   // the leading bit weighs 2^a_lead
    int p_lsb = a_lead - 23 > -149 ? a_lead - 23 : -149;
    const int b_lsb = p_lsb + 298;                // >= 149: rounding bits are integer bits of Q
    uint32_t sig = 0;
    for (int p = L; p >= b_lsb; --p) sig = (sig << 1) | (uint32_t)big_getbit(big, p);
    const int rb = big_getbit(big, b_lsb - 1);
    bool sticky = rem != 0;
    const int below = b_lsb - 1;                  // bits [0, below) are sticky
    for (int i = 0; i < (below >> 5) && !sticky; ++i) sticky = big[i] != 0;
    if (!sticky && (below & 31)) sticky = (big[below >> 5] & ((1u << (below & 31)) - 1u)) != 0;
    if (rb && (sticky || (sig & 1u))) ++sig;      // round half to even
    if (sig == (1u << 24)) {
        sig >>= 1;
        ++p_lsb;
    }
    if (p_lsb + 23 > 127) return INFINITY;
    if (sig < (1u << 23)) return __uint_as_float(sig);   // subnormal: p_lsb == -149
    return __uint_as_float(((uint32_t)(p_lsb + 23 + 127) << 23) | (sig & 0x7fffffu));
}

// ---- the windowed exact sum (the first exact tier)
//
// With T the exponent index of the row's largest |x| (|x| = sig * 2^(t - 149)),
// every square sig^2 * 2^(2t - 298) is a whole number of units
// u = 2^(2T - 354) when t >= T - 28: sig^2 * 2^(2(t - T) + 56) < 2^104, and
// K <= 2^21 of them sum below 2^125.  Squares of elements more than 2^28
// below the largest keep their whole units and flag the dropped remainder
// ("lost"), which adds less than one unit each.
struct U128 {
    uint64_t lo, hi;
};

__host__ __device__ inline void add128(U128& a, uint64_t lo, uint64_t hi) {
    a.lo += lo;
    a.hi += hi + (a.lo < lo ? 1u : 0u);
}

__host__ __device__ inline void window_add(U128& acc, bool& lost, float v, int T) {
    const uint32_t bits = __float_as_uint(v) & 0x7fffffffu;
    const uint32_t e = bits >> 23, f = bits & 0x7fffffu;
    const uint64_t sig = e ? (f | 0x800000u) : f;
    if (!sig) return;
    const int t = e ? (int)e - 1 : 0;
    const uint64_t sq = sig * sig;   // < 2^48
    const int sh = 2 * (t - T) + 56;  // <= 56 (t <= T)
    if (sh >= 0) {
        add128(acc, sq << sh, sh == 0 ? 0ull : sq >> (64 - sh));
    } else if (sh > -48) {
        const uint64_t q = sq >> -sh;
        if ((q << -sh) != sq) lost = true;
        add128(acc, q, 0ull);
    } else {
        lost = true;
    }
}

__host__ __device__ inline int bit128(uint64_t hi, uint64_t lo, int p) {
    if (p < 0 || p >= 128) return 0;
    return p < 64 ? (int)((lo >> p) & 1u) : (int)((hi >> (p - 64)) & 1u);
}

// Whether any bit of (hi, lo) below position p is set.
__host__ __device__ inline bool any_below128(uint64_t hi, uint64_t lo, int p) {
    if (p <= 0) return false;
    if (p >= 128) return (hi | lo) != 0;
    if (p <= 64) return (lo & (p == 64 ? ~0ull : ((1ull << p) - 1ull))) != 0;
    return lo != 0 || (hi & ((1ull << (p - 64)) - 1ull)) != 0;
}

// The float32 nearest (ties to even) to (Q + f) * 2^E for an integer Q >= 1
// and a fraction f in [0, 1) that is zero exactly when sticky_extra is false.
__host__ __device__ inline float round_units(uint64_t qhi, uint64_t qlo, int E, bool sticky_extra) {
    const int L = qhi ? 128 - __builtin_clzll(qhi) : 64 - __builtin_clzll(qlo);   // bit length, >= 1
    const int a_lead = L - 1 + E;
    if (a_lead > 127) return INFINITY;
    int p_lsb = a_lead - 23 > -149 ? a_lead - 23 : -149;
    const int b = p_lsb - E;   // bit of Q that is the float's last significand bit
    uint32_t sig = 0;
    for (int p = L - 1; p >= b && p >= 0; --p) sig = (sig << 1) | (uint32_t)bit128(qhi, qlo, p);
    // b >= 12 here: S holds at least one square of >= 2^56 units, so Q >= 2^35.
    const int rb = bit128(qhi, qlo, b - 1);
    const bool sticky = sticky_extra || any_below128(qhi, qlo, b - 1);
    if (rb && (sticky || (sig & 1u))) ++sig;
    if (sig == (1u << 24)) {
        sig >>= 1;
        ++p_lsb;
    }
    if (p_lsb + 23 > 127) return INFINITY;
    if (sig < (1u << 23)) return __uint_as_float(sig);   // subnormal: p_lsb == -149
    return __uint_as_float(((uint32_t)(p_lsb + 23 + 127) << 23) | (sig & 0x7fffffu));
}

// The exactly rounded mean from the window sum S (units u = 2^E) over K
// terms; false when the dropped remainders could decide the rounding.
__host__ __device__ inline bool window_mean_f32(U128 S, bool lost, uint64_t K, int E, float& out) {
    if ((S.hi | S.lo) == 0) {
        if (lost) return false;
        out = 0.0f;
        return true;
    }
    // Q = floor(S / K), R = S mod K, 32 bits at a time (R < K <= 2^21).
    const uint32_t limb[4] = {(uint32_t)(S.hi >> 32), (uint32_t)S.hi, (uint32_t)(S.lo >> 32), (uint32_t)S.lo};
    uint32_t q[4];
    uint64_t r = 0;
    for (int i = 0; i < 4; ++i) {
        const uint64_t cur = (r << 32) | limb[i];
        q[i] = (uint32_t)(cur / K);
        r = cur % K;
    }
    const uint64_t qhi = ((uint64_t)q[0] << 32) | q[1], qlo = ((uint64_t)q[2] << 32) | q[3];
    if ((qhi | qlo) == 0) return false;   // mean below one unit: leave it to the bins
    if (!lost) {   // exact: S / K = Q + R / K
        out = round_units(qhi, qlo, E, r != 0);
        return true;
    }
    // S / K lies in (Q, Q + 2) units: decided when both ends round alike.
    const uint64_t q1lo = qlo + 1, q1hi = qhi + (q1lo == 0 ? 1u : 0u);
    const float lo_end = round_units(qhi, qlo, E, true), hi_end = round_units(q1hi, q1lo, E, true);
    if (__float_as_uint(lo_end) != __float_as_uint(hi_end)) return false;
    out = lo_end;
    return true;
}

__device__ inline void window_add4(U128& acc, bool& lost, float4 v, int T) {
    window_add(acc, lost, v.x, T);
    window_add(acc, lost, v.y, T);
    window_add(acc, lost, v.z, T);
    window_add(acc, lost, v.w, T);
}

__device__ inline U128 wave_sum128(U128 v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint64_t lo = __shfl_xor(v.lo, off, 64), hi = __shfl_xor(v.hi, off, 64);
        add128(v, lo, hi);
    }
    return v;
}

__device__ inline void bin_square(unsigned long long (*bins)[2], float v) {
    const uint32_t bits = __float_as_uint(v) & 0x7fffffffu;
    const uint32_t e = bits >> 23, f = bits & 0x7fffffu;
    const uint64_t sig = e ? (f | 0x800000u) : f;
    if (!sig) return;
    const int t = e ? ((int)e - 1 < kBins ? (int)e - 1 : kBins - 1) : 0;   // Inf/NaN stay in range
    const uint64_t sq = sig * sig;
    atomicAdd(&bins[t][0], (unsigned long long)(sq >> 24));
    atomicAdd(&bins[t][1], (unsigned long long)(sq & 0xffffffull));
}

__device__ inline void bin_square4(unsigned long long (*bins)[2], float4 v) {
    bin_square(bins, v.x);
    bin_square(bins, v.y);
    bin_square(bins, v.z);
    bin_square(bins, v.w);
}

__device__ inline double sq_sum4(float4 v) {
    const double a = v.x, b = v.y, c = v.z, d = v.w;
    return a * a + b * b + c * c + d * d;   // each square exact; the sum rounds
}

__device__ inline float4 mul4(float4 v, float s) {
    return make_float4(__fmul_rn(v.x, s), __fmul_rn(v.y, s), __fmul_rn(v.z, s), __fmul_rn(v.w, s));
}

// One row of K floats (K % 4 == 0, 16-byte aligned).  R float4 per thread stay
// in registers between the passes; R == 0 re-reads x.
template <int THREADS, int R>
__device__ void rmsnorm_quant_row(const float* __restrict__ x, int64_t K, int8_t* __restrict__ xq,
                                  float* __restrict__ eta_out, int32_t* __restrict__ xsum_out,
                                  float* __restrict__ ms_out) {
    constexpr int W = THREADS / 64;
    __shared__ float redf[W];
    __shared__ double redd[W];
    __shared__ int redi[W];
    __shared__ unsigned long long bins[kBins][2];
    __shared__ uint32_t big[kLimbs];
    __shared__ unsigned long long raw[kLimbs];
    __shared__ float ms_sh;
    __shared__ int ok_sh;
    __shared__ unsigned long long red_lo[W], red_hi[W];
    __shared__ int red_lost[W];
    const float4* x4 = reinterpret_cast<const float4*>(x);
    uint32_t* q4 = reinterpret_cast<uint32_t*>(xq);
    const int64_t n4 = K >> 2;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;

    float amax = 0.0f;
    double ss = 0.0;
    float4 cache[R > 0 ? R : 1];
    if constexpr (R > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t i = t + (int64_t)r * THREADS;
            cache[r] = i < n4 ? x4[i] : make_float4(0, 0, 0, 0);   // plain loads: 3-5% faster at prefill sizes
            const float4 v = cache[r];
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            ss += sq_sum4(v);
        }
    } else {
        for (int64_t i = t; i < n4; i += THREADS) {
            const float4 v = x4[i];
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
            ss += sq_sum4(v);
        }
    }
    amax = wave_max(amax);
    ss = wave_sum_f64(ss);
    if (lane == 0) {
        redf[wave] = amax;
        redd[wave] = ss;
    }
    __syncthreads();
    amax = redf[0];
    ss = redd[0];
#pragma unroll
    for (int w = 1; w < W; ++w) {
        amax = fmaxf(amax, redf[w]);
        ss += redd[w];
    }

    // Fast path: the float64 estimate decides the rounding unless it lies near
    // a boundary.  Every thread evaluates the same test on the same values.
    const double Kd = (double)K;
    const double q = ss / Kd;
    float ms = (float)q;
    const double d = (Kd + 4.0) * 0x1p-52;
    double lo, hi;
    f32_rounding_interval(ms, lo, hi);
    const bool ambiguous = !(q - q * d > lo && q + q * d < hi);
    bool resolved = !ambiguous;
    if (ambiguous) {   // uniform: the windowed exact sum
        const uint32_t ab = __float_as_uint(amax);
        const int T = (ab >> 23) ? (int)(ab >> 23) - 1 : 0;
        U128 acc{0ull, 0ull};
        bool lost = false;
        if constexpr (R > 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (t + (int64_t)r * THREADS < n4) window_add4(acc, lost, cache[r], T);
        } else {
            for (int64_t i = t; i < n4; i += THREADS) window_add4(acc, lost, x4[i], T);
        }
        acc = wave_sum128(acc);
        const bool lost_w = __any(lost);
        if (lane == 0) {
            red_lo[wave] = acc.lo;
            red_hi[wave] = acc.hi;
            red_lost[wave] = lost_w ? 1 : 0;
        }
        __syncthreads();
        if (t == 0) {
            U128 S{0ull, 0ull};
            bool any_lost = false;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                add128(S, red_lo[w], red_hi[w]);
                any_lost = any_lost || red_lost[w];
            }
            float m = 0.0f;
            const bool ok = window_mean_f32(S, any_lost, (uint64_t)K, 2 * T - 354, m);
            ms_sh = m;
            ok_sh = ok ? 1 : 0;
        }
        __syncthreads();
        resolved = ok_sh != 0;
        ms = ms_sh;
    }
    if (!resolved) {   // uniform: the binned exact path
        for (int i = t; i < 2 * kBins; i += THREADS) (&bins[0][0])[i] = 0ull;
        __syncthreads();
        if constexpr (R > 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (t + (int64_t)r * THREADS < n4) bin_square4(bins, cache[r]);
        } else {
            for (int64_t i = t; i < n4; i += THREADS) bin_square4(bins, x4[i]);
        }
        __syncthreads();
        exact_limbs(bins, big, raw, t);
        if (t == 0) ms_sh = exact_mean_f32(big, (uint64_t)K);
        __syncthreads();
        ms = ms_sh;
    }

    const float norm = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, kRmsEps)));
    const float an = __fmul_rn(amax, norm);
    const float eta = an < kScaleFloor ? kScaleFloor : an;
    const float rcp = quant_recip(eta);

    int sum = 0;
    if constexpr (R > 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t i = t + (int64_t)r * THREADS;
            if (i < n4) __builtin_nontemporal_store(quant4(mul4(cache[r], norm), eta, rcp, sum), q4 + i);
        }
    } else {
        for (int64_t i = t; i < n4; i += THREADS) __builtin_nontemporal_store(quant4(mul4(x4[i], norm), eta, rcp, sum), q4 + i);
    }
    if (t == 0) {
        eta_out[0] = eta;
        if (ms_out) ms_out[0] = ms;
    }
    if (xsum_out) {
        sum = wave_sum(sum);
        if (lane == 0) redi[wave] = sum;
        __syncthreads();
        if (t == 0) {
            int s = 0;
#pragma unroll
            for (int w = 0; w < W; ++w) s += redi[w];
            xsum_out[0] = s;
        }
    }
}

template <int THREADS, int R>
__global__ __launch_bounds__(THREADS) void rmsnorm_quant_rows_kernel(
    const float* __restrict__ x, int64_t K, int8_t* __restrict__ xq, float* __restrict__ eta,
    int32_t* __restrict__ xsum, float* __restrict__ ms) {
    const int64_t m = blockIdx.x;
    rmsnorm_quant_row<THREADS, R>(x + m * K, K, xq + m * K, eta + m, xsum ? xsum + m : nullptr,
                                  ms ? ms + m : nullptr);
}

int launch_rmsnorm_quantize(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                            int32_t* xsum, float* ms, hipStream_t stream) {
    if (M == 0) return BITLINEAR_OK;
    const int64_t n4 = K / 4;
    dim3 grid((unsigned)M);
#define BL_RL(T, R) \
    hipLaunchKernelGGL((rmsnorm_quant_rows_kernel<T, R>), grid, dim3(T), 0, stream, x, K, xq, eta, xsum, ms)
    if (n4 <= 256) BL_RL(256, 1);
    else if (n4 <= 512) BL_RL(256, 2);
    else if (n4 <= 1024) BL_RL(256, 4);
    else if (n4 <= 2048) BL_RL(256, 8);
    else if (n4 <= 4096) BL_RL(512, 8);
    else if (n4 <= 8192) BL_RL(1024, 8);
    else BL_RL(1024, 0);
#undef BL_RL
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

}  // namespace bl
