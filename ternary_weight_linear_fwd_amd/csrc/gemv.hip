// gemv.hip -- decode contraction for M <= 4 tokens on gfx950 (VALU dot4 path).
//
// The multiplication-free contraction ([P1] "The MatMul-Free Breakthrough";
// [P2] "3. Additive Integer Accumulation": add on +1, subtract on -1, skip on
// 0) evaluated four weights per instruction.  With code c = w + 1 in {0, 1, 2}
// (the packed 2-bit value itself):
//     sum_{w=+1} x - sum_{w=-1} x  =  sum_k x_k * c_k  -  sum_k x_k,
// exact in int32.  v_dot4 against a code byte adds x twice (+1), once (0) or
// not at all (-1); one sum of x over the same k-range per unit then turns
// that into the add/subtract result.
//
// Work unit: one wavefront owns 64 consecutive output rows (lane = row) and a
// range of k-blocks.  Each k-block is one 16-byte load per lane, i.e. a
// contiguous, 1 KB wave load of the packed layout.  Code fields are taken with
// masks in place (field j of every byte at once: (w >> 2j) & 0x03030303, or
// w & (0x03030303 << 2j) with the 4^j scale folded into a separate
// accumulator), so one packed word costs 5 VALU ops + 4 dot4 per token.  The
// activation bytes are wave-uniform and come from scalar loads.
#include "kernels.hpp"
#include "xcd.hpp"

namespace bl {

constexpr int kGemvWaves = 4;  // wavefronts (work units) per workgroup

template <int M>
struct Acc {
    int a0[M], a1[M], a2[M];
};

// Accumulate one k-block (16 bytes of codes per lane) for M token rows.
template <int M>
__device__ __forceinline__ void dot_block(Acc<M>& acc, const uint4 w, cint4_ptr xs, int64_t xstride,
                                          int64_t kb, int ndw) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if (d >= ndw) break;
        const uint32_t c0 = wd[d] & 0x03030303u;          // field 0: k_local 0..3
        const uint32_t c1 = wd[d] & 0x0C0C0C0Cu;          // field 1 (x4): 4..7
        const uint32_t c2 = wd[d] & 0x30303030u;          // field 2 (x16): 8..11
        const uint32_t c3 = (wd[d] >> 6) & 0x03030303u;   // field 3: 12..15
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const nv_i32x4 x = xs[m * xstride + kb * 4 + d];  // 16 activation bytes
            acc.a0[m] = __builtin_amdgcn_sdot4(x.x, (int)c0, acc.a0[m], false);
            acc.a1[m] = __builtin_amdgcn_sdot4(x.y, (int)c1, acc.a1[m], false);
            acc.a2[m] = __builtin_amdgcn_sdot4(x.z, (int)c2, acc.a2[m], false);
            acc.a0[m] = __builtin_amdgcn_sdot4(x.w, (int)c3, acc.a0[m], false);
        }
    }
}

__device__ inline int wave_sum_i32(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum of xq[m][k] over k in [k0, k1) (a multiple of 4 wide), all lanes.
__device__ inline int xq_range_sum(const int8_t* xrow, int64_t k0, int64_t k1) {
    const int* x = reinterpret_cast<const int*>(xrow);
    int s = 0;
    const int lane = threadIdx.x & 63;
    for (int64_t i = k0 / 4 + lane; i < k1 / 4; i += 64)
        s = __builtin_amdgcn_sdot4(x[i], 0x01010101, s, false);
    return wave_sum_i32(s);
}

struct GemvArgs {
    Problem p;              // single-problem mode
    SplitK sk;
    const Problem* problems;  // grouped mode
    const Unit* units;        // K-slices of a 64-row group in adjacent units
    int32_t* gpart;           // grouped, K split: [unit][M][64] int32 partial sums
    int64_t nunits;
};

template <int M, bool GROUPED, int U>
__global__ __launch_bounds__(256) void gemv_dot4_kernel(GemvArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // Each XCD streams a contiguous run of the units (adjacent weight rows).
    const int64_t u = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * kGemvWaves + wave;
    if (u >= a.nunits) return;

    Problem p;
    int64_t g, kb0, kb1, slice = 0;
    if constexpr (GROUPED) {
        const Unit un = a.units[u];
        p = a.problems[un.problem];
        g = un.group;
        kb0 = 0;
        kb1 = p.Kb;
        if (p.slices > 1) {
            slice = u - p.unit_begin - g * p.slices;
            const int64_t kbs = (p.Kb + p.slices - 1) / p.slices;
            kb0 = slice * kbs;
            kb1 = kb0 + kbs < p.Kb ? kb0 + kbs : p.Kb;
        }
    } else {
        p = a.p;
        const int S = a.sk.S;
        g = u / S;
        slice = u - g * S;
        kb0 = slice * a.sk.kb_per_slice;
        kb1 = kb0 + a.sk.kb_per_slice;
        if (kb1 > p.Kb) kb1 = p.Kb;
    }
    const int64_t K = p.K, N = p.N;
    const int64_t kfull = K / 64;              // complete k-blocks
    const int64_t kend = kb1 < kfull ? kb1 : kfull;
    const int64_t row = g * 64 + lane;

    const uint4* wp = p.packed + (g * p.Kb) * 64 + lane;
    const cint4_ptr xs = as_const(reinterpret_cast<const nv_i32x4*>(p.xq));
    const int64_t xstride = K / 16;            // int4 per token row

    Acc<M> acc;
#pragma unroll
    for (int m = 0; m < M; ++m) acc.a0[m] = acc.a1[m] = acc.a2[m] = 0;

    // Main loop: batches of U complete k-blocks, the next batch in flight
    // while the current one is consumed.
    int64_t kb = kb0;
    if (kb + U <= kend) {
        uint4 cur[U];
#pragma unroll
        for (int i = 0; i < U; ++i) cur[i] = ldnt_u4(wp + (kb + i) * 64);
        for (; kb + U <= kend; kb += U) {
            uint4 nxt[U];
            const bool more = kb + 2 * U <= kend;
            if (more) {
#pragma unroll
                for (int i = 0; i < U; ++i) nxt[i] = ldnt_u4(wp + (kb + U + i) * 64);
            }
#pragma unroll
            for (int i = 0; i < U; ++i) dot_block<M>(acc, cur[i], xs, xstride, kb + i, 4);
            if (more) {
#pragma unroll
                for (int i = 0; i < U; ++i) cur[i] = nxt[i];
            }
        }
    }
    for (; kb < kend; ++kb) dot_block<M>(acc, ldnt_u4(wp + kb * 64), xs, xstride, kb, 4);
    // Partial last block (K % 64 in {16, 32, 48}): only its valid words.
    if (kb1 > kfull && kb0 <= kfull && (K & 63)) {
        dot_block<M>(acc, ldnt_u4(wp + kfull * 64), xs, xstride, kfull,
                     (int)((K & 63) >> 4));
    }

    const int64_t k0 = kb0 * 64, k1 = (kb1 * 64 < K) ? kb1 * 64 : K;
    int res[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const int xsum = xq_range_sum(p.xq + m * K, k0, k1);
        res[m] = acc.a0[m] + (acc.a1[m] >> 2) + (acc.a2[m] >> 4) - xsum;
    }

    if (row >= N) return;
    if (GROUPED && p.slices > 1) {
#pragma unroll
        for (int m = 0; m < M; ++m) a.gpart[(u * M + m) * 64 + lane] = res[m];
        return;
    }
    if (!GROUPED && a.sk.S > 1) {
#pragma unroll
        for (int m = 0; m < M; ++m) a.sk.partial[(slice * M + m) * N + row] = res[m];
        return;
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float s = dequant_scale(p.eta[m], p.gamma);
        p.y[m * N + row] = dequant(res[m], s);
        if (p.y_int) p.y_int[m * N + row] = res[m];
    }
}

// Sum the split-K partials in slice order and apply the dequant epilogue.
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(const int32_t* __restrict__ partial,
                                                              int S, int64_t M, int64_t N,
                                                              const float* __restrict__ eta,
                                                              float gamma, float* __restrict__ y,
                                                              int32_t* __restrict__ y_int) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N) return;
    const int64_t m = i / N;
    int acc = 0;
    for (int s = 0; s < S; ++s) acc += partial[s * M * N + i];
    y[i] = dequant(acc, dequant_scale(eta[m], gamma));
    if (y_int) y_int[i] = acc;
}

int launch_splitk_epilogue(const int32_t* partial, int S, int64_t M, const Problem& p,
                           hipStream_t stream) {
    hipLaunchKernelGGL(splitk_epilogue_kernel, dim3((unsigned)ceil_div(M * p.N, 256)), dim3(256), 0,
                       stream, partial, S, M, (int64_t)p.N, p.eta, p.gamma, p.y, p.y_int);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int gemv_split_slices(int64_t M, int64_t N, int64_t K) {
    (void)M;
    const int64_t G = ceil_div(N, 64), Kb = ceil_div(K, 64);
    int64_t S = ceil_div(1024, G);            // aim for ~1024 wavefronts
    const int64_t max_s = Kb / 4 > 1 ? Kb / 4 : 1;  // at least 4 k-blocks per slice
    if (S > max_s) S = max_s;
    if (S > 16) S = 16;
    if (S < 1) S = 1;
    return (int)S;
}

size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const int S = gemv_split_slices(M, N, K);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

template <int M>
static void launch_single(const GemvArgs& a, int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL((gemv_dot4_kernel<M, false, 4>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
}

int launch_gemv(const Problem& p, int64_t M, void* ws, hipStream_t stream) {
    GemvArgs a{};
    a.p = p;
    const int S = gemv_split_slices(M, p.N, p.K);
    const int64_t Kb = p.Kb;
    a.sk.S = S;
    a.sk.kb_per_slice = (int32_t)ceil_div(Kb, S);
    a.sk.S = (int)ceil_div(Kb, a.sk.kb_per_slice);  // no empty slices
    a.sk.partial = a.sk.S > 1 ? (int32_t*)ws : nullptr;
    a.nunits = ceil_div(p.N, 64) * a.sk.S;
    const int64_t blocks = ceil_div(a.nunits, kGemvWaves);
    switch (M) {
        case 1: launch_single<1>(a, blocks, stream); break;
        case 2: launch_single<2>(a, blocks, stream); break;
        case 3: launch_single<3>(a, blocks, stream); break;
        case 4: launch_single<4>(a, blocks, stream); break;
        default: return BITLINEAR_EUNSUPPORTED;
    }
    BL_LAUNCH_CHECK();
    if (a.sk.S > 1) return launch_splitk_epilogue(a.sk.partial, a.sk.S, M, p, stream);
    return BITLINEAR_OK;
}

template <int M>
static void launch_grouped(const GemvArgs& a, int64_t blocks, hipStream_t stream) {
    // Eight k-blocks per batch (8 KB per wavefront in flight): the grouped
    // launch is one long stream, where the deeper queue pays.
    hipLaunchKernelGGL((gemv_dot4_kernel<M, true, 8>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
}

int launch_gemv_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                        int32_t* partial, hipStream_t stream) {
    GemvArgs a{};
    a.problems = problems;
    a.units = units;
    a.gpart = partial;
    a.nunits = nunits;
    const int64_t blocks = ceil_div(nunits, kGemvWaves);
    switch (M) {
        case 1: launch_grouped<1>(a, blocks, stream); break;
        case 2: launch_grouped<2>(a, blocks, stream); break;
        case 3: launch_grouped<3>(a, blocks, stream); break;
        case 4: launch_grouped<4>(a, blocks, stream); break;
        default: return BITLINEAR_EUNSUPPORTED;
    }
    BL_LAUNCH_CHECK();
    return partial ? launch_grouped_splitk_epilogue(problems, units, nunits, M, 64, partial, stream) : BITLINEAR_OK;
}

}  // namespace bl
