// lut.hip -- compact base-3 weights and the lookup-table decode contraction.
//
// Base-3 format.  [P2] (bandwidth paragraph before "Scaling Laws and
// Empirical Benchmarks": 1.58 bits per weight under compact ternary packing,
// 2 bits otherwise) and [P3] "Common Misconceptions" (log2(3) bits of
// information per weight).  Five weights per byte: digit d = w + 1, canonical
// value v = sum_j d_j 3^j <= 242, 1.6 bits per weight.  Device layout: 64-row
// groups x blocks of 80 k; a block is 1024 bytes, 16 per row, and byte p of a
// row holds k = 80b + 5p + j at 3^j (rows past N and k past K hold digit 1).
// The stored byte is the fraction form q = ceil(256 v / 243), a bijection of
// 0..242 onto 243 of the 256 byte values with v = floor(243 q / 256), from
// which the matrix-core decode takes digits by multiplying by 3 (base3.hip).
//
// Lookup-table contraction.  [P3] "What Most People Miss" (precompute every
// possible outcome of a small block of int8 activations against ternary
// weights, then look the answer up instead of computing it); [P5] "Kernel
// Implementation: The Lookup Table Approach" (weights processed in packed
// groups).  A weight byte covers a group of activations -- five consecutive k
// in the base-3 layout, four k at stride 4 in the 2-bit layout -- and its
// value indexes a table of the group's partial sums:
//     T_g[v] = sum_j (digit_j(v) - 1) * xq[k_g(j)],
// so the contraction is one table read and one add per weight byte, with no
// digit extraction.  Per 64-row block and token a workgroup builds the 16
// tables of the block in LDS (int16: |T| <= 5 * 127), each thread writing
// aligned runs of entries whose low digits count up (9 entries of base 3, 16
// of the 2-bit code) with one add each; then every lane adds the table entries
// its row's 16 bytes select.  One lane owns one row of each of its wavefront's
// RW row groups, so a block's table build is shared by 4 * RW * 64 rows.
#include "lut.hpp"
#include "pack.hpp"
#include "ternary.hpp"

namespace bl {

// ------------------------------------------------------------------ base-3 layout
size_t packed3_bytes(int64_t N, int64_t K) {
    return (size_t)(ceil_div(N, 64) * ceil_div(K, kBase3BlockK) * 1024);
}

struct Pos3 {
    int64_t n, k0;
};

// Dword i of the layout: 4 bytes of one row, k0 .. k0 + 19.
__device__ inline Pos3 pos3(int64_t i, int64_t Kb3) {
    const int64_t q = i & 3, r = (i >> 2) & 63, gb = i >> 8;
    const int64_t g = gb / Kb3, b = gb - g * Kb3;
    return {g * 64 + r, b * kBase3BlockK + q * 20};
}

// Four base-3 bytes from 20 digits (byte c holds digits 5c .. 5c + 4), each
// in the fraction form.
__device__ inline uint32_t pack3_dword(const uint32_t (&d)[20]) {
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t v = d[5 * c] + 3 * d[5 * c + 1] + 9 * d[5 * c + 2] + 27 * d[5 * c + 3] +
                           81 * d[5 * c + 4];
        word |= base3_fraction_byte(v) << (8 * c);
    }
    return word;
}

__global__ __launch_bounds__(256) void ternarize_pack3_kernel(const float* __restrict__ W, int64_t N,
                                                              int64_t K, int64_t Kb3,
                                                              const float* __restrict__ gamma_p,
                                                              uint32_t* __restrict__ packed,
                                                              int64_t ndwords) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= ndwords) return;
    const Pos3 p = pos3(i, Kb3);
    uint32_t d[20];
#pragma unroll
    for (int q = 0; q < 20; ++q) d[q] = 1u;   // pad: zero weight
    if (p.n < N) {
        const float gamma = gamma_p[0];
#pragma unroll
        for (int q = 0; q < 20; ++q)
            if (p.k0 + q < K) d[q] = ternary_code(W[p.n * K + p.k0 + q], gamma);
    }
    packed[i] = pack3_dword(d);
}

__global__ __launch_bounds__(256) void pack3_ternary_kernel(const int8_t* __restrict__ Wt, int64_t N,
                                                            int64_t K, int64_t Kb3,
                                                            uint32_t* __restrict__ packed,
                                                            int64_t ndwords, int32_t* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= ndwords) return;
    const Pos3 p = pos3(i, Kb3);
    uint32_t d[20];
    int nbad = 0;
#pragma unroll
    for (int q = 0; q < 20; ++q) {
        d[q] = 1u;
        if (p.n < N && p.k0 + q < K) {
            const int w = Wt[p.n * K + p.k0 + q];
            const bool ok = w >= -1 && w <= 1;
            nbad += !ok;
            d[q] = ok ? (uint32_t)(w + 1) : 1u;
        }
    }
    packed[i] = pack3_dword(d);
    if (nbad && bad) atomicAdd(bad, nbad);
}

__global__ __launch_bounds__(256) void unpack3_kernel(const uint32_t* __restrict__ packed, int64_t N,
                                                      int64_t K, int64_t Kb3, int8_t* __restrict__ Wt,
                                                      int64_t ndwords, int32_t* __restrict__ bad) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= ndwords) return;
    const Pos3 p = pos3(i, Kb3);
    if (p.n >= N || p.k0 >= K) return;
    const uint32_t word = packed[i];
    int nbad = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t q = (word >> (8 * c)) & 0xffu;
        uint32_t v = base3_canonical_byte(q);
        const int64_t kc = p.k0 + 5 * c;
        if (kc >= K) break;
        const bool ok = base3_fraction_byte(v) == q;   // 13 byte values are no fraction form
        nbad += !ok;
        if (!ok) v = 121u;   // decoded as zero weights
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            const uint32_t q3 = (v * 171u) >> 9;   // v / 3 for v < 256
            const int digit = (int)(v - 3u * q3);
            v = q3;
            if (kc + j < K) Wt[p.n * K + kc + j] = (int8_t)(digit - 1);
        }
    }
    if (nbad && bad) atomicAdd(bad, nbad);
}

static int64_t layout3_dwords(int64_t N, int64_t K) {
    return ceil_div(N, 64) * ceil_div(K, kBase3BlockK) * 256;
}

int launch_pack_weights3(const float* W, int64_t N, int64_t K, uint8_t* packed3, float* gamma_dev,
                         void* ws, hipStream_t stream) {
    // gamma exactly as the 2-bit packer computes it (its workspace layout)
    int rc = launch_gamma(W, N, K, gamma_dev, ws, stream);
    if (rc) return rc;
    const float* gamma_ws = (const float*)((const char*)ws + kGammaBins * sizeof(unsigned long long));
    const int64_t nd = layout3_dwords(N, K);
    hipLaunchKernelGGL(ternarize_pack3_kernel, dim3((unsigned)ceil_div(nd, 256)), dim3(256), 0, stream,
                       W, N, K, ceil_div(K, kBase3BlockK), gamma_ws, (uint32_t*)packed3, nd);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_pack_ternary3(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed3, int32_t* bad,
                         hipStream_t stream) {
    const int64_t nd = layout3_dwords(N, K);
    hipLaunchKernelGGL(pack3_ternary_kernel, dim3((unsigned)ceil_div(nd, 256)), dim3(256), 0, stream,
                       Wt, N, K, ceil_div(K, kBase3BlockK), (uint32_t*)packed3, nd, bad);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_unpack3(const uint8_t* packed3, int64_t N, int64_t K, int8_t* Wt, int32_t* bad,
                   hipStream_t stream) {
    const int64_t nd = layout3_dwords(N, K);
    hipLaunchKernelGGL(unpack3_kernel, dim3((unsigned)ceil_div(nd, 256)), dim3(256), 0, stream,
                       (const uint32_t*)packed3, N, K, ceil_div(K, kBase3BlockK), Wt, nd, bad);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

// ------------------------------------------------------------------ lookup tables
template <int FMT>
struct LutFmt;

// 2-bit layout: block of 64 k; byte p of a row's 16 bytes is byte i = p & 3 of
// word d = p >> 2, whose 2-bit field j is k = 16d + i + 4j.
template <>
struct LutFmt<kFormat2Bit> {
    static constexpr int BK = 64;
    static constexpr int RUN = 16;    // entries per run: the two low fields
    static constexpr int RUNS = 16;   // runs per table (256 entries)
    __device__ static int k_of(int p, int j) { return 16 * (p >> 2) + (p & 3) + 4 * j; }
};

// Base-3 layout: block of 80 k; byte p holds k = 5p + j at 3^j.
template <>
struct LutFmt<kFormatBase3> {
    static constexpr int BK = 80;
    static constexpr int RUN = 9;     // entries per run: the two low digits
    static constexpr int RUNS = 27;   // runs per table (243 entries at their stored bytes; 13 stay 0)
    __device__ static int k_of(int p, int j) { return 5 * p + j; }
};

struct LutArgs {
    Problem p;        // p.packed: the format's layout
    int32_t* partial; // [S][M][N] split-K partial sums, or null when S == 1
    int64_t M;
    int32_t Kb;       // blocks of the format along K
    int32_t S;        // k-slices
    int32_t kb_per_slice;
    int32_t row_wgs;  // workgroups along N
};

// Build the 16 tables of block b for tokens m0 .. m0 + MC - 1 (xs holds their
// activations of the block, 0 past K).
template <int FMT, int MC>
__device__ inline void build_tables(int16_t (*tab)[16][256], const int (*xs)[80], int mc) {
    using F = LutFmt<FMT>;
    constexpr int TASKS = 16 * F::RUNS;
    for (int task = threadIdx.x; task < TASKS * mc; task += 256) {
        const int mm = task / TASKS, rest = task - mm * TASKS;
        const int p = rest / F::RUNS, u = rest - p * F::RUNS;
        const int x0 = xs[mm][F::k_of(p, 0)], x1 = xs[mm][F::k_of(p, 1)];
        const int x2 = xs[mm][F::k_of(p, 2)], x3 = xs[mm][F::k_of(p, 3)];
        if constexpr (FMT == kFormatBase3) {
            const int x4 = xs[mm][F::k_of(p, 4)];
            // canonical value 9u + 3 d1 + d0: high digits from u, low digits
            // counting up; the entry sits at its stored (fraction-form) byte
            const int d2 = u % 3, d3 = (u / 3) % 3, d4 = u / 9;
            const int base = (d2 - 1) * x2 + (d3 - 1) * x3 + (d4 - 1) * x4 - x0 - x1;
            int16_t* tb = &tab[mm][p][0];
#pragma unroll
            for (int d1 = 0; d1 < 3; ++d1)
#pragma unroll
                for (int d0 = 0; d0 < 3; ++d0)
                    tb[base3_fraction_byte(9u * u + 3u * d1 + d0)] = (int16_t)(base + d1 * x1 + d0 * x0);
        } else {
            // entry 16u + 4 f1 + f0: fields 2 and 3 from u; field 3 (never
            // produced) only needs a bounded value
            const int f2 = u & 3, f3 = u >> 2;
            int16_t* t = &tab[mm][p][u * F::RUN];
            const int base = (f2 - 1) * x2 + (f3 - 1) * x3 - x0 - x1;
#pragma unroll
            for (int f1 = 0; f1 < 4; ++f1)
#pragma unroll
                for (int f0 = 0; f0 < 4; ++f0) t[4 * f1 + f0] = (int16_t)(base + f1 * x1 + f0 * x0);
        }
    }
}

template <int FMT, int MC, int RW>
__global__ __launch_bounds__(256) void lut_gemv_kernel(LutArgs a) {
    using F = LutFmt<FMT>;
    __shared__ int16_t tab[MC][16][256];
    __shared__ int xs[MC][80];
    const Problem& p = a.p;
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int64_t rwg = blockIdx.x % a.row_wgs, slice = blockIdx.x / a.row_wgs;
    const int64_t G = ceil_div((int64_t)p.N, 64), K = p.K, N = p.N, M = a.M;
    const int64_t kb0 = slice * a.kb_per_slice;
    int64_t kb1 = kb0 + a.kb_per_slice;
    if (kb1 > a.Kb) kb1 = a.Kb;
    const uint4* packed = p.packed;

    // The 13 entries of a base-3 table at bytes that are no fraction form
    // are never written by the builder.
    if constexpr (FMT == kFormatBase3)
        for (int i = t; i < MC * 16 * 256; i += 256) {
            const uint32_t q = (uint32_t)i & 255u;
            if (base3_fraction_byte(base3_canonical_byte(q)) != q) tab[i >> 12][(i >> 8) & 15][q] = 0;
        }

    int64_t g_of[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) g_of[i] = (rwg * 4 + wave) * RW + i;

    for (int64_t m0 = 0; m0 < M; m0 += MC) {
        const int mc = M - m0 < MC ? (int)(M - m0) : MC;
        int acc[RW][MC];
#pragma unroll
        for (int i = 0; i < RW; ++i)
#pragma unroll
            for (int mm = 0; mm < MC; ++mm) acc[i][mm] = 0;

        for (int64_t b = kb0; b < kb1; ++b) {
            // this block's weight chunks, in flight while the tables are built
            uint4 w[RW];
#pragma unroll
            for (int i = 0; i < RW; ++i)
                w[i] = g_of[i] < G ? ldnt_u4(packed + (g_of[i] * a.Kb + b) * 64 + lane)
                                   : make_uint4(0, 0, 0, 0);
            __syncthreads();   // every lane is done with the previous block's tables
            for (int i = t; i < mc * F::BK; i += 256) {
                const int mm = i / F::BK, kk = i - mm * F::BK;
                const int64_t k = b * F::BK + kk;
                xs[mm][kk] = k < K ? (int)p.xq[(m0 + mm) * K + k] : 0;
            }
            __syncthreads();
            build_tables<FMT, MC>(tab, xs, mc);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < RW; ++i) {
                const uint32_t wv[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const uint32_t v = (wv[q >> 2] >> (8 * (q & 3))) & 0xffu;
#pragma unroll
                    for (int mm = 0; mm < MC; ++mm)
                        if (mm < mc) acc[i][mm] += tab[mm][q][v];
                }
            }
        }

#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const int64_t n = g_of[i] * 64 + lane;
            if (n >= N) continue;
#pragma unroll
            for (int mm = 0; mm < MC; ++mm) {
                if (mm >= mc) continue;
                const int64_t m = m0 + mm;
                if (a.S > 1) {
                    a.partial[(slice * M + m) * N + n] = acc[i][mm];
                } else {
                    p.y[m * N + n] = dequant(acc[i][mm], dequant_scale(p.eta[m], p.gamma));
                    if (p.y_int) p.y_int[m * N + n] = acc[i][mm];
                }
            }
        }
    }
}

constexpr int kLutRW = 8;   // row groups per wavefront: 2048 rows per workgroup

struct LutPlan {
    int64_t row_wgs, Kb;
    int S, kb_per_slice;
};

static LutPlan lut_plan(int64_t M, int64_t N, int64_t K, int format) {
    (void)M;
    LutPlan pl;
    pl.Kb = ceil_div(K, format == kFormatBase3 ? (int64_t)kBase3BlockK : (int64_t)64);
    pl.row_wgs = ceil_div(ceil_div(N, 64), (int64_t)4 * kLutRW);
    int64_t S = ceil_div((int64_t)512, pl.row_wgs);   // aim for ~512 workgroups
    if (S > pl.Kb) S = pl.Kb;
    if (S > 64) S = 64;
    if (S < 1) S = 1;
    pl.kb_per_slice = (int)ceil_div(pl.Kb, S);
    pl.S = (int)ceil_div(pl.Kb, (int64_t)pl.kb_per_slice);
    return pl;
}

size_t lut_ws_bytes(int64_t M, int64_t N, int64_t K, int format) {
    const LutPlan pl = lut_plan(M, N, K, format);
    return pl.S > 1 ? (size_t)pl.S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

template <int FMT>
static void launch_lut_fmt(const LutArgs& a, int64_t blocks, hipStream_t stream) {
    if (a.M >= 4)
        hipLaunchKernelGGL((lut_gemv_kernel<FMT, 4, kLutRW>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else if (a.M >= 2)
        hipLaunchKernelGGL((lut_gemv_kernel<FMT, 2, kLutRW>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((lut_gemv_kernel<FMT, 1, kLutRW>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
}

int launch_lut(const Problem& p, int64_t M, int format, void* ws, hipStream_t stream) {
    if (M == 0) return BITLINEAR_OK;
    const LutPlan pl = lut_plan(M, p.N, p.K, format);
    LutArgs a{};
    a.p = p;
    a.M = M;
    a.Kb = (int32_t)pl.Kb;
    a.S = pl.S;
    a.kb_per_slice = pl.kb_per_slice;
    a.row_wgs = (int32_t)pl.row_wgs;
    a.partial = pl.S > 1 ? (int32_t*)ws : nullptr;
    const int64_t blocks = pl.row_wgs * pl.S;
    if (format == kFormatBase3) launch_lut_fmt<kFormatBase3>(a, blocks, stream);
    else launch_lut_fmt<kFormat2Bit>(a, blocks, stream);
    BL_LAUNCH_CHECK();
    if (pl.S > 1) return launch_splitk_epilogue(a.partial, pl.S, M, p, stream);
    return BITLINEAR_OK;
}

}  // namespace bl
