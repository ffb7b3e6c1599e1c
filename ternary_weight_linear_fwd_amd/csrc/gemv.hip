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
#include "quant_row.hpp"
#include "xcd.hpp"

namespace bl {


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

    // Main loop over the complete k-blocks of the range: a ring of U
    // registers, each refilled with the block U further on right after its
    // use, so U loads stay in flight all along.  The loads go through a
    // buffer descriptor on exactly those blocks (wave-uniform, in scalar
    // registers): one past the end returns zeros without touching memory, so
    // every load is issued unconditionally and the compiler waits for one
    // block at a time.
    const int rk0 = __builtin_amdgcn_readfirstlane((int)kb0);
    const int run = __builtin_amdgcn_readfirstlane((int)(kend > kb0 ? kend - kb0 : 0));
    {
        const uint8_t* wrun = uniform_ptr(reinterpret_cast<const uint8_t*>(p.packed + (g * p.Kb + rk0) * 64));
        const __amdgpu_buffer_rsrc_t wres =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wrun), 0, run * 1024, kBufferRsrcWord3);
        const int wl = lane * 16;
        auto wload = [&](int j) {   // block rk0 + j (zeros past the range)
            // The whole offset in the vector operand, which the range check
            // covers.
            const nv_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wres, wl + j * 1024, 0, kLoadNonTemporal);
            return make_uint4(v.x, v.y, v.z, v.w);
        };
        uint4 wq[U];
#pragma unroll
        for (int i = 0; i < U; ++i) wq[i] = wload(i);
        const int rounds = (run + U - 1) / U;
        for (int r = 0; r + 1 < rounds; ++r) {   // every block of these rounds is inside the range
#pragma unroll
            for (int i = 0; i < U; ++i) {
                dot_block<M>(acc, wq[i], xs, xstride, rk0 + r * U + i, 4);
                wq[i] = wload((r + 1) * U + i);
                // Each refill right after its slot's use (the scheduler would
                // gather them at the end of the round).
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (rounds > 0) {
            const int last = (rounds - 1) * U;
#pragma unroll
            for (int i = 0; i < U; ++i)
                if (last + i < run) dot_block<M>(acc, wq[i], xs, xstride, rk0 + last + i, 4);
        }
    }
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

// ---- fused decode (M <= 4: small grouped plans, short single calls)
//
// A plan too small to fill the chip (one transformer block at a few tokens:
// 520 row groups for hidden 3200 / FFN 8640) gives each (problem, 64-row
// group) one workgroup of kFusedWaves wavefronts that covers the whole K
// loop: wavefront w streams a contiguous run of the group's k-blocks (all of
// its loads in flight at once up to kFusedBatch blocks).  Before contracting,
// the workgroup quantizes the problem's M activation rows itself with the
// quantizer's own arithmetic ([P1] "2. Absmax Dynamic Activation
// Quantization": eta = max(max_k |x|, 1e-5), x~ = clamp(rne((x * 127) / eta),
// -128, 127)) into LDS, along with each row's sum of x~; every workgroup of a
// problem reads the same rows (from L2 after the first) and reaches the same
// bits.  The wavefronts' partial sums meet in LDS and one pass subtracts
// sum x~, dequantizes and stores.  The workgroup of row group 0 also writes
// x~ and eta to the problem's xq / eta buffers, as the separate quantize stage
// would.  No second launch, no partial sums in memory.
constexpr int kFusedWaves = 8;
constexpr int kFusedThreads = 64 * kFusedWaves;
// k-blocks in flight per wavefront (registers: up to two tokens six
// wavefronts per SIMD, so that three 8-wave workgroups fit on a CU; three
// and four tokens four, two workgroups)
template <int M>
constexpr int fused_batch() { return M == 1 ? 12 : 8; }
constexpr int kFusedChunks = kFusedMaxK / 4 / kFusedThreads;   // float4 of a row per thread


// Accumulate one k-block (16 bytes of codes per lane) against x~ rows in LDS
// (row m at xs + m * kpad; every lane reads the same bytes: a broadcast).
template <int M>
__device__ __forceinline__ void dot_block_lds(Acc<M>& acc, const uint4 w, const uint8_t* xs, int64_t kpad,
                                              int64_t kb) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t c0 = wd[d] & 0x03030303u;
        const uint32_t c1 = wd[d] & 0x0C0C0C0Cu;
        const uint32_t c2 = wd[d] & 0x30303030u;
        const uint32_t c3 = (wd[d] >> 6) & 0x03030303u;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const nv_i32x4 x = *reinterpret_cast<const nv_i32x4*>(xs + m * kpad + kb * 64 + d * 16);
            acc.a0[m] = __builtin_amdgcn_sdot4(x.x, (int)c0, acc.a0[m], false);
            acc.a1[m] = __builtin_amdgcn_sdot4(x.y, (int)c1, acc.a1[m], false);
            acc.a2[m] = __builtin_amdgcn_sdot4(x.z, (int)c2, acc.a2[m], false);
            acc.a0[m] = __builtin_amdgcn_sdot4(x.w, (int)c3, acc.a0[m], false);
        }
    }
}

// SINGLE: one problem given by value (x = NULL: x~ and eta given), row group
// = blockIdx.x; otherwise (problem, row group) from the grouped table.
template <int M, bool SINGLE>
__global__ __launch_bounds__(kFusedThreads, M <= 2 ? 6 : 4) void gemv_fused_kernel(const Problem* __restrict__ problems,
                                                                   const Unit* __restrict__ units, int64_t nunits,
                                                                   Problem single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];   // [M][Kb * 64] x~, zero at k >= K
    __shared__ float red_max[M][kFusedWaves];
    __shared__ int red_sum[M][kFusedWaves];
    __shared__ int xsum_sh[M];
    __shared__ float eta_sh[M];
    __shared__ int part[kFusedWaves][M][64];

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63;
    // Units in table order (longest K first), which the dispatcher deals
    // round-robin to the XCDs: problems of different K (the long down
    // projection) spread evenly over the XCDs' shares of memory bandwidth.
    const Problem p = SINGLE ? single : problems[units[blockIdx.x].problem];
    const int64_t K = p.K, N = p.N, Kb = p.Kb, g = SINGLE ? (int64_t)blockIdx.x : (int64_t)units[blockIdx.x].group;
    const int64_t kpad = Kb * 64;

    // This wavefront's contiguous run of k-blocks.
    const int64_t nbw = (Kb + kFusedWaves - 1) / kFusedWaves;
    const int64_t kb0 = (int64_t)wave * nbw;
    const int64_t kb1 = kb0 + nbw < Kb ? kb0 + nbw : Kb;

    // x~ rows into LDS, with eta and sum x~ per row (the float32 chunks and the
    // weight words below are never live together: registers for occupancy).
    const int64_t n4 = K >> 2;
#pragma unroll 1
    for (int m = 0; m < M; ++m) {
        uint32_t* q4 = reinterpret_cast<uint32_t*>(xs + m * kpad);
        int sum = 0;
        if (p.x) {
            const float4* x4 = reinterpret_cast<const float4*>(p.x + m * K);
            float4 v[kFusedChunks];
            float amax = 0.0f;
#pragma unroll
            for (int r = 0; r < kFusedChunks; ++r) {
                const int64_t i = t + (int64_t)r * kFusedThreads;
                v[r] = i < n4 ? ldg_f4(x4 + i) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[r].x), fabsf(v[r].y)), fmaxf(fabsf(v[r].z), fabsf(v[r].w))));
            }
            amax = wave_max(amax);
            if (lane == 0) red_max[m][wave] = amax;
            __syncthreads();
            amax = red_max[m][0];
#pragma unroll
            for (int w = 1; w < kFusedWaves; ++w) amax = fmaxf(amax, red_max[m][w]);
            const float eta = amax < kScaleFloor ? kScaleFloor : amax;
            const float rcp = quant_recip(eta);
#pragma unroll
            for (int r = 0; r < kFusedChunks; ++r) {
                const int64_t i = t + (int64_t)r * kFusedThreads;
                if (i < n4) q4[i] = quant4(v[r], eta, rcp, sum);
            }
            if (t == 0) eta_sh[m] = eta;
        } else {
            // Already quantized: copy x~ (16 bytes per thread and pass) and sum it.
            const uint4* src = reinterpret_cast<const uint4*>(p.xq + m * K);
            for (int64_t i = t; i < K / 16; i += kFusedThreads) {
                const uint4 v = src[i];
                reinterpret_cast<uint4*>(q4)[i] = v;
                sum = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, sum, false);
                sum = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, sum, false);
                sum = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, sum, false);
                sum = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, sum, false);
            }
            if (t == 0) eta_sh[m] = p.eta[m];
        }
        // k in [K, kpad): zero activations against the pad codes.
        for (int64_t i = n4 + t; i < kpad / 4; i += kFusedThreads) q4[i] = 0u;
        sum = wave_sum(sum);
        if (lane == 0) red_sum[m][wave] = sum;
    }
    __syncthreads();
    if (t < M) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < kFusedWaves; ++w) s += red_sum[t][w];
        xsum_sh[t] = s;
    }

    __syncthreads();   // x~, eta and the row sums are in LDS (a full barrier: no loads in flight here)

    // The run's k-blocks, up to kFusedBatch in flight, through a buffer
    // descriptor on exactly the run: the run bounds and the group's weight
    // rows are the same for every lane (scalar registers), and a load past
    // the run returns zeros without touching memory.  So every load is
    // issued unconditionally and the compiler counts the loads in flight
    // exactly, waiting for one block at a time.
    constexpr int kFusedBatch = fused_batch<M>();
    const int rb0 = __builtin_amdgcn_readfirstlane((int)kb0);
    const int run = __builtin_amdgcn_readfirstlane((int)(kb1 > kb0 ? kb1 - kb0 : 0));
    const uint8_t* wrun = uniform_ptr(reinterpret_cast<const uint8_t*>(p.packed + (g * Kb + rb0) * 64));
    const __amdgpu_buffer_rsrc_t wres =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wrun), 0, run * 1024, kBufferRsrcWord3);
    const int wl = lane * 16;
    auto wload = [&](int j) {   // block rb0 + j of the run (zeros past its end)
        // The whole offset in the vector operand, which the range check
        // covers.
        const nv_u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wres, wl + j * 1024, 0, kLoadNonTemporal);
        return make_uint4(v.x, v.y, v.z, v.w);
    };
    // Nothing is in flight here (the barrier above follows the last
    // activation load); saying so keeps the compiler from carrying a load it
    // cannot see completed on some path (one thread's eta read) into the
    // weight loads, where it would wait for all of them.
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    uint4 wq[kFusedBatch];
#pragma unroll
    for (int i = 0; i < kFusedBatch; ++i) wq[i] = wload(i);

    Acc<M> acc;
#pragma unroll
    for (int m = 0; m < M; ++m) acc.a0[m] = acc.a1[m] = acc.a2[m] = 0;
    // The registers form a ring: as soon as slot i's block has been used the
    // slot is refilled with the block kFusedBatch further on, so a run longer
    // than one batch keeps kFusedBatch loads in flight instead of waiting a
    // second memory round trip for its tail.  Every block of a round before
    // the last lies inside the run.
    const int rounds = (run + kFusedBatch - 1) / kFusedBatch;
    for (int r = 0; r + 1 < rounds; ++r) {
#pragma unroll
        for (int i = 0; i < kFusedBatch; ++i) {
            dot_block_lds<M>(acc, wq[i], xs, kpad, rb0 + r * kFusedBatch + i);
            wq[i] = wload((r + 1) * kFusedBatch + i);
            // Keep each refill right after its slot's use: left to itself the
            // scheduler gathers the refills at the end of the round, which
            // turns the ring back into batches.
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (rounds > 0) {
        const int last = (rounds - 1) * kFusedBatch;
#pragma unroll
        for (int i = 0; i < kFusedBatch; ++i)
            if (last + i < run) dot_block_lds<M>(acc, wq[i], xs, kpad, rb0 + last + i);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) part[wave][m][lane] = acc.a0[m] + (acc.a1[m] >> 2) + (acc.a2[m] >> 4);
    __syncthreads();

    if (t < 64 * M) {
        const int m = t >> 6;
        const int64_t row = g * 64 + lane;
        int v = 0;
#pragma unroll
        for (int w = 0; w < kFusedWaves; ++w) v += part[w][m][lane];
        v -= xsum_sh[m];
        if (row < N) {
            p.y[m * N + row] = dequant(v, dequant_scale(eta_sh[m], p.gamma));
            if (p.y_int) p.y_int[m * N + row] = v;
        }
    }

    // Row group 0 hands x~ and eta on, as the quantize stage does.
    if (g == 0 && p.x) {
        for (int m = 0; m < M; ++m) {
            const uint4* src = reinterpret_cast<const uint4*>(xs + m * kpad);
            uint4* dst = reinterpret_cast<uint4*>(const_cast<int8_t*>(p.xq) + m * K);
            for (int64_t i = t; i < K / 16; i += kFusedThreads) dst[i] = src[i];
            if (t == 0) const_cast<float*>(p.eta)[m] = eta_sh[m];
        }
    }
}

int launch_gemv_fused(const Problem* problems, const Unit* units, int64_t nunits, int64_t M, int64_t max_K,
                      hipStream_t stream) {
    if (max_K > kFusedMaxK) return BITLINEAR_EUNSUPPORTED;
    const size_t lds = (size_t)M * (size_t)(ceil_div(max_K, 64) * 64);
    const dim3 grid((unsigned)nunits), block(kFusedThreads);
    const Problem none{};
    switch (M) {
        case 1:
            hipLaunchKernelGGL((gemv_fused_kernel<1, false>), grid, block, lds, stream, problems, units, nunits, none);
            break;
        case 2:
            hipLaunchKernelGGL((gemv_fused_kernel<2, false>), grid, block, lds, stream, problems, units, nunits, none);
            break;
        case 3:
            hipLaunchKernelGGL((gemv_fused_kernel<3, false>), grid, block, lds, stream, problems, units, nunits, none);
            break;
        case 4:
            hipLaunchKernelGGL((gemv_fused_kernel<4, false>), grid, block, lds, stream, problems, units, nunits, none);
            break;
        default: return BITLINEAR_EUNSUPPORTED;
    }
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

// A single problem of at most kFusedMaxM tokens runs the fused kernel -- one
// workgroup per 64-row group whose wavefronts split the K loop and meet in
// LDS, no split-K partials and no second launch -- where each wavefront's
// run of k-blocks is one batch of loads, or two on a grid of at least
// kFusedSingleGroups groups, and the x~ rows fit the LDS.  Measured on
// MI355X against the split GEMV and its epilogue (graph replay, weights
// cycled): 2048 x 2048 at one token 5.5 -> 4.0 us, 8640 x 3200 7.0 -> 5.1,
// 28672 x 8192 16.4 -> 14.2, at four tokens 31.6 -> 20.7; the long-K runs
// it leaves to the split GEMV (8192 x 28672 16.2 against 19.4 fused;
// 1024 x 8192 6.3 against 6.9).
constexpr int64_t kFusedSingleGroups = 32;
constexpr int64_t kFusedSingleMaxLds = 32 * 1024;

bool gemv_fused_single(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || M > kFusedMaxM || M * ceil_div(K, 64) * 64 > kFusedSingleMaxLds) return false;
    const int64_t run = ceil_div(ceil_div(K, 64), kFusedWaves);   // k-blocks per wavefront
    return run <= 8 || (run <= 16 && ceil_div(N, 64) >= kFusedSingleGroups);
}

int launch_gemv_fused_single(const Problem& p, int64_t M, hipStream_t stream) {
    if (p.x && p.K > kFusedMaxK) return BITLINEAR_EUNSUPPORTED;
    const size_t lds = (size_t)M * (size_t)(p.Kb * 64);
    const dim3 grid((unsigned)ceil_div(p.N, 64)), block(kFusedThreads);
    switch (M) {
        case 1: hipLaunchKernelGGL((gemv_fused_kernel<1, true>), grid, block, lds, stream, nullptr, nullptr, 0, p); break;
        case 2: hipLaunchKernelGGL((gemv_fused_kernel<2, true>), grid, block, lds, stream, nullptr, nullptr, 0, p); break;
        case 3: hipLaunchKernelGGL((gemv_fused_kernel<3, true>), grid, block, lds, stream, nullptr, nullptr, 0, p); break;
        case 4: hipLaunchKernelGGL((gemv_fused_kernel<4, true>), grid, block, lds, stream, nullptr, nullptr, 0, p); break;
        default: return BITLINEAR_EUNSUPPORTED;
    }
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

// Sum the split-K partials and apply the dequant epilogue.  One output per
// lane in 64-lane workgroups (a 28672-wide row is 448 of them), each lane
// with up to 32 partial loads in flight at once (one memory round trip for
// the slice counts the planners choose): the sum is exact in int32, so its
// order does not matter.
constexpr int kEpiLoads = 32;

__global__ __launch_bounds__(64) void splitk_epilogue_kernel(const int32_t* __restrict__ partial,
                                                             int S, int64_t M, int64_t N,
                                                             const float* __restrict__ eta,
                                                             float gamma, float* __restrict__ y,
                                                             int32_t* __restrict__ y_int) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    const int64_t MN = M * N;
    if (i >= MN) return;
    const int64_t m = i / N;
    const float sc = dequant_scale(eta[m], gamma);   // its load goes out before the partials'
    int acc = 0;
    for (int s0 = 0; s0 < S; s0 += kEpiLoads) {
        int v[kEpiLoads];
#pragma unroll
        for (int j = 0; j < kEpiLoads; ++j) v[j] = s0 + j < S ? partial[(s0 + j) * MN + i] : 0;
#pragma unroll
        for (int j = 0; j < kEpiLoads; ++j) acc += v[j];
    }
    y[i] = dequant(acc, sc);
    if (y_int) y_int[i] = acc;
}

int launch_splitk_epilogue(const int32_t* partial, int S, int64_t M, const Problem& p,
                           hipStream_t stream) {
    hipLaunchKernelGGL(splitk_epilogue_kernel, dim3((unsigned)ceil_div(M * p.N, 64)), dim3(64), 0,
                       stream, partial, S, M, (int64_t)p.N, p.eta, p.gamma, p.y, p.y_int);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int gemv_split_slices(int64_t M, int64_t N, int64_t K) {
    (void)M;
    const int64_t G = ceil_div(N, 64), Kb = ceil_div(K, 64);
    // aim for ~4096 wavefronts (16 per CU): a lone projection is too short a
    // stream for fewer to keep enough loads in flight (measured 19.4 -> 16.3
    // us for 8192 -> 28672 and 21.5 -> 16.4 us for 28672 -> 8192 at one token)
    int64_t S = ceil_div(4096, G);
    const int64_t max_s = Kb / 4 > 1 ? Kb / 4 : 1;  // at least 4 k-blocks per slice
    if (S > max_s) S = max_s;
    if (S > 16) S = 16;
    if (S < 1) S = 1;
    return (int)S;
}

size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K) {
    if (gemv_fused_single(M, N, K)) return 0;
    const int S = gemv_split_slices(M, N, K);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

template <int M>
static void launch_single(const GemvArgs& a, int64_t blocks, hipStream_t stream) {
    hipLaunchKernelGGL((gemv_dot4_kernel<M, false, 4>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, a);
}

int launch_gemv(const Problem& p, int64_t M, void* ws, hipStream_t stream) {
    if (!p.x && gemv_fused_single(M, p.N, p.K)) return launch_gemv_fused_single(p, M, stream);
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
