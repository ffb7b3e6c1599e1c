/*
 * bitlinear_oracle.c -- plain, slow CPU oracle for the BitNet b1.58 BitLinear
 * forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or constant with the GPU
 * library: every constant below is declared here again on purpose.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -shared -fPIC
 *        (no -ffast-math: every float operation must be the IEEE one written).
 *
 * Sources, cited by page title and section:
 *  [P1] "BitNet b1.58 & 1-Bit LLMs in Production: Ternary Quantization,
 *       MatMul-Free Kernels, and Edge AI Silicon Deployment"
 *  [P2] "1-Bit Large Language Models and BitNet b1.58: How Ternary Weights and
 *       Additive Kernels Eliminate Matrix Multiplications"
 *  [P4] "BitNet b1.58 & 1-Bit LLM Architectures: Eliminating Matrix
 *       Multiplication and Running 70B Models on CPU in 2026"
 *  [P5] "BitNet b1.58: Ternary Weight LLMs That Eliminate Matrix
 *       Multiplication"
 *
 * Readings taken where the pages are silent or disagree (each is listed with
 * its reason in the design notes of the repository):
 *  - gamma is the exact mean of |W| over the whole matrix, rounded once to the
 *    nearest float32 (ties to even), then clamped below at 1e-5.  The pages give
 *    the mean as a formula and leave its evaluation order open.
 *  - Rounding is round-half-to-even everywhere (the listings use torch.round).
 *  - Activation scale: eta = max(max_k |x[m][k]|, 1e-5) per token row m;
 *    xq = clamp(rne((x * 127) / eta), -128, 127), multiply first, then an IEEE
 *    float32 division, as both code listings write it.
 *  - Dequant: s = (eta * gamma) / 127 in float32, y = float(y_int) * s.
 *  - Canonical 2-bit code: -1 -> 00, 0 -> 01, +1 -> 10; weight j of a byte sits
 *    in bits 2j..2j+1; a row holds ceil(K/4) bytes and pads with code 01.
 *  - RMSNorm (the optional step before quantization): the mean of x^2 is the
 *    exact mean rounded once to float32; norm = 1 / sqrt(ms + 1e-6) as an IEEE
 *    square root and an IEEE division; x_norm = x * norm.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <pthread.h>

#define OR_QB 127.0f          /* Q_b of the activation quantizer          */
#define OR_SCALE_FLOOR 1e-5f  /* lower clamp on eta and gamma             */

/* ------------------------------------------------------------------------ */
/* Exact arithmetic on non-negative integers held as little-endian 32-bit    */
/* limbs.  Used only by the gamma and mean-of-squares computations.          */
/* ------------------------------------------------------------------------ */
#define OR_LIMBS 20 /* 640 bits: the exact sum of up to 2^40 |floats| needs 318
                       bits, of up to 2^31 squared floats 586 */

typedef struct { uint32_t w[OR_LIMBS]; } or_big;

static void big_zero(or_big* a) { memset(a, 0, sizeof(*a)); }

/* a += v * 2^shift, v < 2^32 */
static void big_add_shifted(or_big* a, uint32_t v, int shift) {
    int limb = shift / 32, bit = shift % 32;
    uint64_t carry = ((uint64_t)v) << bit; /* at most 63 bits */
    for (int i = limb; i < OR_LIMBS && carry; ++i) {
        uint64_t s = (uint64_t)a->w[i] + (carry & 0xffffffffu);
        a->w[i] = (uint32_t)s;
        carry = (carry >> 32) + (s >> 32);
    }
}

static int big_bitlen(const or_big* a) {
    for (int i = OR_LIMBS - 1; i >= 0; --i)
        if (a->w[i]) {
            int b = 32;
            while (!(a->w[i] & (1u << (b - 1)))) --b;
            return i * 32 + b;
        }
    return 0;
}

static int big_bit(const or_big* a, int pos) {
    if (pos < 0 || pos >= OR_LIMBS * 32) return 0;
    return (a->w[pos / 32] >> (pos % 32)) & 1u;
}

/* 1 if any bit of a below position pos is set */
static int big_any_below(const or_big* a, int pos) {
    for (int i = 0; i < pos && i < OR_LIMBS * 32; ++i)
        if (big_bit(a, i)) return 1;
    return 0;
}

/*
 * The float32 nearest to S * 2^unit / D (S a non-negative big integer, D in
 * [1, 2^40)), ties to even, with subnormal results and overflow to +Inf.
 * Plain long division, one quotient bit at a time from the top: the first
 * quotient 1 fixes the exponent and with it the last significand position
 * (23 places lower, but never below the 2^-149 subnormal step); the next bit
 * rounds, and every bit after it, with the final remainder, is sticky.
 */
static float big_ratio_to_f32(const or_big* S, int unit, uint64_t D) {
    const int L = big_bitlen(S);
    if (L == 0) return 0.0f;
    uint64_t rem = 0, sig = 0;
    int started = 0, p_lsb = 0, rb = 0, sticky = 0;
    for (int pos = L - 1;; --pos) {
        rem = (rem << 1) | (uint64_t)big_bit(S, pos);   /* zero bits once pos < 0 */
        int qb = 0;
        if (rem >= D) { rem -= D; qb = 1; }
        const int a = pos + unit;                       /* this quotient bit weighs 2^a */
        if (!started) {
            if (a <= -151) return 0.0f;                 /* below half the smallest subnormal */
            if (!qb) continue;
            started = 1;
            p_lsb = a - 23 > -149 ? a - 23 : -149;
        }
        if (a >= p_lsb) {
            sig = (sig << 1) | (uint64_t)qb;
        } else if (a == p_lsb - 1) {
            rb = qb;
            sticky = rem != 0 || big_any_below(S, pos);
            break;
        }
    }
    if (rb && (sticky || (sig & 1u))) ++sig;             /* round half to even */
    if (sig == (1u << 24)) { sig >>= 1; ++p_lsb; }       /* carry into the next binade */
    if (p_lsb + 23 > 127) return INFINITY;               /* beyond the largest float32 */
    return (float)ldexp((double)sig, p_lsb);             /* exact: sig < 2^24, in range */
}

/*
 * Absmean weight scale.
 * [P1] section "1. Absmean Weight Quantization" (gamma = mean of |W_ij| over
 * the n x m matrix) and the WeightQuantizerSTE listing in "Production PyTorch
 * Implementation: BitLinear b1.58 Layer" (clamp at 1e-5); [P2] "Inside the
 * BitLinear Layer", "1. Absmean Weight Quantization"; [P4] "The Weight
 * Quantization Function: Absmean Scaling".
 *
 * Every finite float32 magnitude is sig * 2^(t - 149) with an integer sig <
 * 2^24 and 0 <= t <= 253, so the sum of all |W| is an exact integer count of
 * 2^-149 units.  The mean S / (N*K) is then rounded to float32 by the exact
 * ratio rounding above.
 */
int oracle_absmean_gamma(const float* W, int64_t N, int64_t K, float* gamma_out) {
    if (!W || !gamma_out || N <= 0 || K <= 0) return -1;
    const uint64_t D = (uint64_t)N * (uint64_t)K;
    if (D >> 40) return -1;
    or_big S;
    big_zero(&S);
    for (uint64_t i = 0; i < D; ++i) {
        uint32_t bits;
        memcpy(&bits, &W[i], 4);
        bits &= 0x7fffffffu;             /* |w| */
        uint32_t e = bits >> 23, f = bits & 0x7fffffu;
        if (e == 255) return -2;         /* Inf/NaN: outside the contract */
        uint32_t sig = e ? (f | 0x800000u) : f;
        int t = e ? (int)e - 1 : 0;      /* |w| = sig * 2^(t-149) */
        if (sig) big_add_shifted(&S, sig, t);
    }
    /* S * 2^-149 / D, rounded once to the nearest float32 (ties to even);
       a subnormal or zero mean falls under the clamp below. */
    float g = big_ratio_to_f32(&S, -149, D);
    if (g < OR_SCALE_FLOOR) g = OR_SCALE_FLOOR;
    *gamma_out = g;
    return 0;
}

/*
 * Absmedian weight scale: the median of |W| over the whole matrix in place of
 * the mean.  [P2] "Scaling Laws and Empirical Benchmarks"
 * (BitNet b1.58 Reloaded: adjusting the quantization baseline to the median,
 * "Absmedian", rather than the mean).  Readings: the median of the N*K
 * magnitudes; for an even count it is the mean of the two middle ones, that
 * mean rounded once to float32 (ties to even); clamped below at 1e-5 like
 * gamma; ternarization then divides by it exactly as with the absmean scale.
 * Non-negative float32 magnitudes order like their bit patterns, so the
 * magnitudes are sorted as unsigned integers.
 */
static int or_cmp_u32(const void* a, const void* b) {
    uint32_t x = *(const uint32_t*)a, y = *(const uint32_t*)b;
    return x < y ? -1 : x > y;
}

int oracle_absmedian_gamma(const float* W, int64_t N, int64_t K, float* gamma_out) {
    if (!W || !gamma_out || N <= 0 || K <= 0) return -1;
    const uint64_t D = (uint64_t)K * (uint64_t)N;   /* entries */
    if (D >> 40) return -1;
    uint32_t* mag = (uint32_t*)malloc(D * sizeof(uint32_t));
    if (!mag) return -6;
    for (uint64_t i = 0; i < D; ++i) {
        uint32_t bits;
        memcpy(&bits, &W[i], 4);
        bits &= 0x7fffffffu;
        if ((bits >> 23) == 255) { free(mag); return -2; }   /* Inf/NaN: outside the contract */
        mag[i] = bits;
    }
    qsort(mag, D, sizeof(uint32_t), or_cmp_u32);
    const uint32_t lo = mag[(D - 1) / 2], hi = mag[D / 2];   /* equal when D is odd */
    free(mag);
    /* (lo + hi) / 2 exactly: both are sig * 2^(t-149); add the two in 2^-149 units */
    or_big S;
    big_zero(&S);
    const uint32_t two[2] = {lo, hi};
    for (int i = 0; i < 2; ++i) {
        uint32_t e = two[i] >> 23, f = two[i] & 0x7fffffu;
        uint32_t sig = e ? (f | 0x800000u) : f;
        int te = e ? (int)e - 1 : 0;
        if (sig) big_add_shifted(&S, sig, te);
    }
    float g = big_ratio_to_f32(&S, -149, 2);
    if (!(g >= OR_SCALE_FLOOR)) g = OR_SCALE_FLOOR;
    *gamma_out = g;
    return 0;
}

/*
 * Ternarization: W~ = Clip(Round(W / gamma), -1, +1).
 * [P1] "1. Absmean Weight Quantization" and the WeightQuantizerSTE listing
 * (division, torch.round, clamp); [P2] "1. Absmean Weight Quantization".
 */
int oracle_ternarize(const float* W, int64_t N, int64_t K, float gamma, int8_t* Wt) {
    if (!W || !Wt || N <= 0 || K <= 0 || !(gamma > 0.0f)) return -1;
    for (int64_t i = 0; i < N * K; ++i) {
        float t = W[i] / gamma;          /* IEEE float32 division */
        float r = nearbyintf(t);         /* round half to even */
        if (r > 1.0f) r = 1.0f;
        if (r < -1.0f) r = -1.0f;
        Wt[i] = (int8_t)r;
    }
    return 0;
}

/*
 * Canonical 2-bit packing, four weights per byte.
 * [P1] "Production Deployment Standards for Edge Systems Engineers", item 1
 * ({-1,0,+1} -> {00,01,10}); [P5] "Kernel Implementation: The Lookup Table
 * Approach" (encoding comment; field j of a byte at bits 2j..2j+1).
 * Row n occupies ceil(K/4) bytes; byte b holds k = 4b + j; pad fields hold 01.
 */
int64_t oracle_packed_row_bytes(int64_t K) { return (K + 3) / 4; }

int oracle_pack(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed) {
    if (!Wt || !packed || N <= 0 || K <= 0) return -1;
    const int64_t rb = oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < rb; ++b) {
            uint8_t byte = 0;
            for (int j = 0; j < 4; ++j) {
                int64_t k = 4 * b + j;
                int code;
                if (k >= K) code = 1;                     /* pad: zero weight */
                else if (Wt[n * K + k] == 1) code = 2;
                else if (Wt[n * K + k] == 0) code = 1;
                else if (Wt[n * K + k] == -1) code = 0;
                else return -3;                           /* not ternary */
                byte |= (uint8_t)(code << (2 * j));
            }
            packed[n * rb + b] = byte;
        }
    return 0;
}

int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wt) {
    if (!Wt || !packed || N <= 0 || K <= 0) return -1;
    const int64_t rb = oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            int code = (packed[n * rb + k / 4] >> (2 * (k % 4))) & 3;
            if (code == 3) return -4;                     /* never produced */
            Wt[n * K + k] = (int8_t)(code - 1);
        }
    return 0;
}

/*
 * Compact ternary packing, five weights per byte (3^5 = 243 <= 256, 1.6 bits
 * per weight).  [P2] "Scaling Laws..." context paragraph on memory bandwidth
 * (1.58 bits per parameter under compact ternary packing, 2 bits otherwise);
 * [P3] "Common Misconceptions" (log2(3) ~ 1.58 bits of information per
 * ternary weight).  The pages name the packing but not its layout; reading
 * taken: digit d = w + 1 in {0, 1, 2} as in the 2-bit code, byte b of row n
 * holds k = 5b + j as the base-3 digit of weight 3^j, v = sum_j d_j 3^j in
 * [0, 242]; a row holds ceil(K/5) bytes and pads with digit 1 (weight 0).
 */
int64_t oracle_packed3_row_bytes(int64_t K) { return (K + 4) / 5; }

int oracle_pack3(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed) {
    if (!Wt || !packed || N <= 0 || K <= 0) return -1;
    const int64_t rb = oracle_packed3_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < rb; ++b) {
            int v = 0, place = 1;
            for (int j = 0; j < 5; ++j, place *= 3) {
                int64_t k = 5 * b + j;
                int digit;
                if (k >= K) digit = 1;                    /* pad: zero weight */
                else if (Wt[n * K + k] == 1) digit = 2;
                else if (Wt[n * K + k] == 0) digit = 1;
                else if (Wt[n * K + k] == -1) digit = 0;
                else return -3;                           /* not ternary */
                v += digit * place;
            }
            packed[n * rb + b] = (uint8_t)v;
        }
    return 0;
}

int oracle_unpack3(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wt) {
    if (!Wt || !packed || N <= 0 || K <= 0) return -1;
    const int64_t rb = oracle_packed3_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < rb; ++b) {
            int v = packed[n * rb + b];
            if (v >= 243) return -4;                      /* never produced */
            for (int j = 0; j < 5; ++j) {
                int digit = v % 3;
                v /= 3;
                int64_t k = 5 * b + j;
                if (k < K) Wt[n * K + k] = (int8_t)(digit - 1);
            }
        }
    return 0;
}

/*
 * Per-token absmax INT8 activation quantization.
 * [P1] "2. Absmax Dynamic Activation Quantization" (Q_b = 127) and the
 * ActivationQuantizerSTE listing (max over the last dim, clamp 1e-5,
 * round(x * 127.0 / eta), clamp to [-128, 127]); [P4] "Activation
 * Quantization: 8-Bit Absmax Scaling"; [P5] bitlinear_forward listing in
 * "Weight Quantization: Absmean Centralization".
 */
int oracle_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta) {
    if (!x || !xq || !eta || M < 0 || K <= 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * K;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > amax) amax = a;
        }
        float e = amax < OR_SCALE_FLOOR ? OR_SCALE_FLOOR : amax;
        eta[m] = e;
        for (int64_t k = 0; k < K; ++k) {
            float scaled = row[k] * OR_QB;   /* x * 127.0 */
            float q = scaled / e;            /* ... / eta, IEEE division */
            float r = nearbyintf(q);         /* round half to even */
            if (r > 127.0f) r = 127.0f;
            if (r < -128.0f) r = -128.0f;
            xq[m * K + k] = (int8_t)r;
        }
    }
    return 0;
}

/*
 * RMSNorm without affine parameters, the step before activation quantization.
 * [P1] pipeline box 1 ("RMSNorm") and step 1 of BitLinear158.forward in
 * "Production PyTorch Implementation: BitLinear b1.58 Layer" (norm = rsqrt of
 * the mean of x^2 over the last dim plus 1e-6; x_norm = x * norm); [P1] "2.
 * Absmax Dynamic Activation Quantization" (normalization without learnable
 * affine parameters precedes the quantizer); [P2] "2. Absmax Activation
 * Quantization" (normalization before quantization).
 *
 * Readings (the pages leave these open):
 *  - the mean of the squares is the exact mean, rounded once to the nearest
 *    float32 (ties to even): every finite float32 is sig * 2^(t - 149), so its
 *    square is sig^2 * 2^(2t - 298) and the row sum is an exact integer count
 *    of 2^-298 units;
 *  - rsqrt is evaluated as two IEEE float32 operations, a square root and a
 *    division: norm = 1 / sqrt(ms + 1e-6), each step rounded to nearest even;
 *  - x_norm = x * norm in float32.
 * ms_out and norm_out (each [M], may be NULL) receive the per-row mean of the
 * squares and the factor.
 */
#define OR_RMS_EPS 1e-6f

int oracle_rmsnorm(const float* x, int64_t M, int64_t K, float* xn, float* ms_out,
                   float* norm_out) {
    if (!x || !xn || M < 0 || K <= 0) return -1;
    if (K >> 40) return -1;
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * K;
        or_big S;
        big_zero(&S);
        for (int64_t k = 0; k < K; ++k) {
            uint32_t bits;
            memcpy(&bits, &row[k], 4);
            bits &= 0x7fffffffu;
            uint32_t e = bits >> 23, f = bits & 0x7fffffu;
            if (e == 255) return -2;                     /* Inf/NaN: outside the contract */
            uint64_t sig = e ? (f | 0x800000u) : f;
            int ex = e ? (int)e - 1 : 0;                 /* |x| = sig * 2^(ex-149) */
            uint64_t sq = sig * sig;                     /* < 2^48: x^2 = sq * 2^(2ex-298) */
            if (sq) {
                big_add_shifted(&S, (uint32_t)(sq & 0xffffffffu), 2 * ex);
                big_add_shifted(&S, (uint32_t)(sq >> 32), 2 * ex + 32);
            }
        }
        const float ms = big_ratio_to_f32(&S, -298, (uint64_t)K);
        const float t = ms + OR_RMS_EPS;                 /* mean + 1e-6 */
        const float s = sqrtf(t);                        /* IEEE square root */
        const float norm = 1.0f / s;                     /* IEEE division */
        for (int64_t k = 0; k < K; ++k) xn[m * K + k] = row[k] * norm;
        if (ms_out) ms_out[m] = ms;
        if (norm_out) norm_out[m] = norm;
    }
    return 0;
}

/* RMSNorm followed by the absmax quantizer on the normalized rows. */
int oracle_rmsnorm_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                                float* ms_out, float* norm_out) {
    if (!x || !xq || !eta || M < 0 || K <= 0) return -1;
    if (M == 0) return 0;
    float* xn = (float*)malloc((size_t)M * (size_t)K * sizeof(float));
    if (!xn) return -6;
    int rc = oracle_rmsnorm(x, M, K, xn, ms_out, norm_out);
    if (!rc) rc = oracle_quantize_act(xn, M, K, xq, eta);
    free(xn);
    return rc;
}

/*
 * The multiplication-free contraction:
 *   y_int[m][n] = sum_{k : W~[n][k] = +1} xq[m][k] - sum_{k : W~[n][k] = -1} xq[m][k]
 * [P1] "The MatMul-Free Breakthrough" (partition of additions and
 * subtractions) and pipeline box 4; [P2] "3. Additive Integer Accumulation"
 * (add on +1, subtract on -1, skip on 0); [P5] "The Arithmetic Collapse".
 * W~ is [N][K] (output-major, as nn.Linear stores it); accumulation is int64
 * and checked to fit int32.
 */
typedef struct {
    const int8_t* xq; const int8_t* Wt; int64_t M, N, K; int32_t* y;
    int64_t n0, n1; int overflow;
} or_contract_job;

static void* or_contract_rows(void* arg) {
    or_contract_job* j = (or_contract_job*)arg;
    for (int64_t m = 0; m < j->M; ++m)
        for (int64_t n = j->n0; n < j->n1; ++n) {
            const int8_t* xr = j->xq + m * j->K;
            const int8_t* wr = j->Wt + n * j->K;
            int64_t plus = 0, minus = 0;
            for (int64_t k = 0; k < j->K; ++k) {
                if (wr[k] == 1) plus += xr[k];
                else if (wr[k] == -1) minus += xr[k];
                /* zero weight: skipped */
            }
            int64_t acc = plus - minus;
            if (acc > INT32_MAX || acc < INT32_MIN) j->overflow = 1;
            j->y[m * j->N + n] = (int32_t)acc;
        }
    return 0;
}

int oracle_ternary_contract(const int8_t* xq, const int8_t* Wt, int64_t M, int64_t N,
                            int64_t K, int32_t* y_int, int threads) {
    if (!xq || !Wt || !y_int || M < 0 || N <= 0 || K <= 0) return -1;
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > N) threads = (int)N;
    or_contract_job jobs[256];
    pthread_t tid[256];
    for (int t = 0; t < threads; ++t) {
        jobs[t].xq = xq; jobs[t].Wt = Wt; jobs[t].M = M; jobs[t].N = N; jobs[t].K = K;
        jobs[t].y = y_int; jobs[t].overflow = 0;
        jobs[t].n0 = N * t / threads; jobs[t].n1 = N * (t + 1) / threads;
    }
    if (threads == 1) or_contract_rows(&jobs[0]);
    else {
        for (int t = 0; t < threads; ++t) pthread_create(&tid[t], 0, or_contract_rows, &jobs[t]);
        for (int t = 0; t < threads; ++t) pthread_join(tid[t], 0);
    }
    for (int t = 0; t < threads; ++t) if (jobs[t].overflow) return -5;
    return 0;
}

/*
 * Dequantization: y = y_int * ((eta * gamma) / 127).
 * [P1] pipeline box 5 and step 5 of BitLinear158.forward (scale =
 * (eta * gamma) / 127.0, output = y_raw * scale); [P5] bitlinear_forward
 * listing (one scalar rescale per token); [P2] "3. Additive Integer
 * Accumulation" (rescale once by beta*gamma/Q_b).
 */
int oracle_dequant(const int32_t* y_int, const float* eta, float gamma, int64_t M,
                   int64_t N, float* y) {
    if (!y_int || !eta || !y || M < 0 || N <= 0) return -1;
    for (int64_t m = 0; m < M; ++m) {
        float eg = eta[m] * gamma;   /* eta * gamma */
        float s = eg / OR_QB;        /* ... / 127.0 */
        for (int64_t n = 0; n < N; ++n) y[m * N + n] = (float)y_int[m * N + n] * s;
    }
    return 0;
}

/*
 * The whole forward from float32 activations and ternary weights with their
 * scale: quantize, contract, dequantize.  xq/eta/y_int may be NULL when the
 * caller does not need the intermediates (they are then kept internally only
 * when provided).  [P1] BitLinear158.forward steps 2, 4 and 5 (step 1, the
 * RMSNorm, and step 3, the weight quantizer, happen outside this call).
 */
int oracle_forward(const float* x, const int8_t* Wt, float gamma, int64_t M, int64_t N,
                   int64_t K, float* y, int8_t* xq, float* eta, int32_t* y_int,
                   int threads) {
    if (!x || !Wt || !y || !xq || !eta || !y_int) return -1;
    int rc = oracle_quantize_act(x, M, K, xq, eta);
    if (rc) return rc;
    rc = oracle_ternary_contract(xq, Wt, M, N, K, y_int, threads);
    if (rc) return rc;
    return oracle_dequant(y_int, eta, gamma, M, N, y);
}
