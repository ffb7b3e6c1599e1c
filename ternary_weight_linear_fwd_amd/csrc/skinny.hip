// skinny.hip -- decode contraction for 4 < M <= 64 tokens on the gfx950
// matrix cores (v_mfma_i32_16x16x64_i8), streaming like the GEMV.
//
// The contraction of [P2] "3. Additive Integer Accumulation" with the same
// identity as the dot4 path: with c = w + 1 in {0, 1, 2} (the packed code),
//     sum_{w=+1} x - sum_{w=-1} x  =  sum_k x_k * c_k  -  sum_k x_k .
// The codes go to the MFMA as they are (field j of a word is
// (w >> 2j) & 0x03030303: 7 VALU ops per 16 weights, no byte permute), and
// one extra MFMA per 16-row tile and 64-k group multiplies the same A
// fragment by an all-ones operand, which yields sum_k x_k for every row in
// the accumulator layout of the output.  Any k whose code is 01 -- pad
// positions inside the last block, or blocks outside a work unit's range
// forced to 01 -- contributes x_k to both terms and cancels exactly, so A may
// be read from clamped addresses there.
//
// Work unit: a workgroup of four wavefronts owns 256 consecutive output rows
// of one problem (each wavefront 64 rows = four 16-column MFMA tiles) and a
// range of k-blocks.  Per K-step (256 k):
//  * the workgroup's 16*MT activation rows x 256 bytes arrive once, by direct
//    global->LDS loads (global_load_lds_dwordx4, 1 KB per wave instruction)
//    into a double-buffered stage; chunk c of row r sits at chunk c ^ (r & 15)
//    so the 16 rows a ds_read_b128 serves hit distinct banks;
//  * each lane loads its four 16-byte weight chunks (row n of each tile,
//    k-block kb + g) into registers -- a wave load is four 256-byte runs of
//    the packed layout -- one step ahead of their use.
// One barrier per step.
#include "kernels.hpp"
#include "xcd.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kSkinnyWaves = kSkinnyRows / 64;

struct SkinnyArgs {
    Problem p;                // single-problem mode
    SplitK sk;
    const Problem* problems;  // grouped mode
    const Unit* units;        // grouped: (problem, 256-row block), K-slices innermost
    int32_t* gpart;           // grouped, K split: [unit][M][256] int32 partial sums
    int64_t nunits;           // work units = workgroups
    int32_t M;
};


// One 16-byte-per-lane direct global->LDS load (the wave's 64 lanes fill 1 KB).
__device__ __forceinline__ void skinny_dma16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

// Queue one K-step (4 k-blocks): the activation stage by direct-to-LDS loads,
// this lane's weight chunks into registers (code 01 past the unit's range).
template <int MT>
__device__ __forceinline__ void skinny_issue(uint8_t* stage, const int8_t* const (&asrc)[MT],
                                             const int (&acol)[MT], const uint4* wrow, uint4 (&bq)[4],
                                             int64_t kb, int64_t kb1, int64_t K, bool group_ok,
                                             int wave, int lg) {
    const int64_t kbase = kb * 64;
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        int64_t off = kbase;
        if (kbase + acol[j] >= K) off = K - 16 - acol[j];   // past K: meets code 01
        skinny_dma16(asrc[j] + off, stage + (j * kSkinnyWaves + wave) * 1024);
    }
    const int64_t kbl = kb + lg;
    const bool in = group_ok && kbl < kb1;
#pragma unroll
    for (int t = 0; t < 4; ++t)
        bq[t] = in ? ldnt_u4(wrow + kbl * 64 + t * 16)
                   : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
}

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256) void skinny_mfma_kernel(SkinnyArgs a) {
    constexpr int ROWS = 16 * MT;          // activation rows of the stage
    constexpr int STAGE = ROWS * 256;      // bytes
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * STAGE];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    Problem p;
    int64_t blk, kb0, kb1, slice = 0;
    // Each XCD streams a contiguous run of the units (adjacent weight rows,
    // adjacent output columns).
    const uint32_t u = xcd_contiguous(blockIdx.x, (uint32_t)a.nunits);
    if constexpr (GROUPED) {
        const Unit un = a.units[u];
        p = a.problems[un.problem];
        blk = un.group;
        kb0 = 0;
        kb1 = p.Kb;
        if (p.slices > 1) {
            slice = (int64_t)u - p.unit_begin - blk * p.slices;
            const int64_t kbs = skinny_slice_kb(p.Kb, p.slices);
            kb0 = slice * kbs;
            kb1 = kb0 + kbs < p.Kb ? kb0 + kbs : p.Kb;
        }
    } else {
        p = a.p;
        const int S = a.sk.S;
        blk = u / S;
        slice = u - blk * S;
        kb0 = slice * a.sk.kb_per_slice;
        kb1 = kb0 + a.sk.kb_per_slice;
        if (kb1 > p.Kb) kb1 = p.Kb;
    }
    const int64_t M = a.M, N = p.N, K = p.K;
    const int64_t g = blk * kSkinnyWaves + wave;         // this wave's 64-row group
    const bool group_ok = g < ceil_div(N, 64);
    const int nl = lane & 15, lg = lane >> 4;
    const uint4* wrow = p.packed + (group_ok ? g : 0) * p.Kb * 64 + nl;

    // DMA sources: physical slot P of a stage holds row P >> 4, chunk (P & 15) ^ row.
    const int8_t* asrc[MT];
    int acol[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int P = (j * kSkinnyWaves + wave) * 64 + lane;
        const int r = P >> 4;
        acol[j] = ((P & 15) ^ (r & 15)) * 16;
        const int64_t m = r < M ? r : M - 1;             // rows past M: never stored
        asrc[j] = p.xq + m * K + acol[j];
    }
    v4i acc[MT][4], accs[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        accs[i] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = v4i{0, 0, 0, 0};
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

    uint4 bcur[4], bnext[4];
    skinny_issue<MT>(lds, asrc, acol, wrow, bcur, kb0, kb1, K, group_ok, wave, lg);
    int st = 0;
    for (int64_t kb = kb0; kb < kb1; kb += 4, st ^= 1) {
        __builtin_amdgcn_s_waitcnt(0);   // this step's activations (LDS) and weights (registers)
        __syncthreads();                 // ... for every wave; the other stage is free
        const bool more = kb + 4 < kb1;
        if (more) skinny_issue<MT>(lds + (st ^ 1) * STAGE, asrc, acol, wrow, bnext, kb + 4, kb1, K, group_ok, wave, lg);
        const uint8_t* A = lds + st * STAGE;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            v4i af[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int r = i * 16 + nl;
                af[i] = *reinterpret_cast<const v4i*>(A + r * 256 + (((lg * 4 + d) ^ (r & 15)) << 4));
            }
#pragma unroll
            for (int i = 0; i < MT; ++i)
                accs[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], ones, accs[i], 0, 0, 0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t w = d == 0 ? bcur[t].x : d == 1 ? bcur[t].y : d == 2 ? bcur[t].z : bcur[t].w;
                v4i bf;
                bf.x = (int)(w & 0x03030303u);
                bf.y = (int)((w >> 2) & 0x03030303u);
                bf.z = (int)((w >> 4) & 0x03030303u);
                bf.w = (int)((w >> 6) & 0x03030303u);
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf, acc[i][t], 0, 0, 0);
            }
        }
        if (more) {
#pragma unroll
            for (int t = 0; t < 4; ++t) bcur[t] = bnext[t];
        }
    }

    const bool split = GROUPED ? p.slices > 1 : a.sk.S > 1;
    if (MT == 1 && !split && !p.y_int && (N & 3) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0) {
        // Up to 16 token rows: the block's 16 x 256 outputs go through LDS (8
        // rows at a time, in the stage buffers, free after the K loop) and
        // leave as whole row runs, 16 bytes per lane and 1 KB per wave store,
        // with non-temporal stores.  Measured 3.7% faster over the 70B-shaped
        // sweep at 16 tokens than per-element device-scope stores.
        float* stage = reinterpret_cast<float*>(lds);   // [8][256]
        const int t = threadIdx.x;
        const int64_t n0 = blk * kSkinnyRows;
        // The scales of this lane's four token rows, their loads issued
        // together (rows past M read row 0 and are never stored).
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = lg * 4 + r;
            sc[r] = dequant_scale(p.eta[m < M ? m : 0], p.gamma);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            __syncthreads();   // the last K step's reads (or the previous half's stores) are done
            if (group_ok) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = lg * 4 + r;
                    if ((m >> 3) != h || m >= M) continue;
#pragma unroll
                    for (int tt = 0; tt < 4; ++tt)
                        stage[(m & 7) * 256 + wave * 64 + tt * 16 + nl] = dequant(acc[0][tt][r] - accs[0][r], sc[r]);
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // A wavefront stores one token row's 1 KB run (row is the
                // same on all its lanes), through a buffer descriptor on that
                // run so that the store can carry the device-scope policy:
                // written through the XCD's L2 at once (1% faster over the
                // 70B-shaped sweep at 16 tokens than non-temporal stores, 3%
                // than plain write-back ones).
                const int row = __builtin_amdgcn_readfirstlane((t >> 6) + 4 * q), c4 = t & 63;
                const int64_t m = 8 * h + row, n = n0 + c4 * 4;
                if (m >= M || n >= N) continue;   // N % 4 == 0: a float4 is wholly inside or outside
                const nv_u32x4 v = *reinterpret_cast<const nv_u32x4*>(stage + row * 256 + c4 * 4);
                __amdgpu_buffer_rsrc_t run = __builtin_amdgcn_make_buffer_rsrc(p.y + m * N + n0, 0, 1024, kBufferRsrcWord3);
                __builtin_amdgcn_raw_buffer_store_b128(v, run, c4 * 16, 0, kStoreDeviceScope);
            }
        }
        return;
    }
    // Epilogue: element r of tile (i, t) is row 16i + 4lg + r, column 16t + nl.
    if (!group_ok) return;
    // The scales of this lane's rows, their loads issued together.
    float sc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = i * 16 + lg * 4 + r;
            sc[i][r] = split ? 0.0f : dequant_scale(p.eta[m < M ? m : 0], p.gamma);
        }
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = i * 16 + lg * 4 + r;
            if (m >= M) continue;
            const float s = sc[i][r];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t n = g * 64 + t * 16 + nl;
                if (n >= N) continue;
                const int v = acc[i][t][r] - accs[i][r];
                if (GROUPED && split) {
                    a.gpart[((int64_t)u * M + m) * kSkinnyRows + (n - blk * kSkinnyRows)] = v;
                } else if (split) {
                    a.sk.partial[(slice * M + m) * N + n] = v;
                } else {
                    // Device-scope stores write through the XCD's L2: the
                    // outputs then leave at once instead of as dirty lines
                    // evicted later into the weight stream (measured faster
                    // at 16 tokens; relaxed, so values and order are those
                    // of plain stores).
                    __hip_atomic_store(p.y + m * N + n, dequant(v, s), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (p.y_int)
                        __hip_atomic_store(p.y_int + m * N + n, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    }
}

int skinny_split_slices(int64_t M, int64_t N, int64_t K) {
    (void)M;
    const int64_t G = ceil_div(N, 64), Kb = ceil_div(K, 64);
    int64_t S = ceil_div(1024, G);                 // aim for ~1024 wavefronts
    const int64_t max_s = Kb / 8 > 1 ? Kb / 8 : 1;  // at least 8 k-blocks (2 steps) per slice
    if (S > max_s) S = max_s;
    if (S > 16) S = 16;
    if (S < 1) S = 1;
    return (int)S;
}

size_t skinny_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const int S = skinny_split_slices(M, N, K);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

template <int MT>
static void launch_skinny_mt(const SkinnyArgs& a, int64_t blocks, bool grouped, hipStream_t stream) {
    if (grouped)
        hipLaunchKernelGGL((skinny_mfma_kernel<MT, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((skinny_mfma_kernel<MT, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
}

static int launch_skinny_any(const SkinnyArgs& a, bool grouped, hipStream_t stream) {
    const int64_t blocks = a.nunits;
    if (a.M <= 16) launch_skinny_mt<1>(a, blocks, grouped, stream);
    else if (a.M <= 32) launch_skinny_mt<2>(a, blocks, grouped, stream);
    else if (a.M <= 48) launch_skinny_mt<3>(a, blocks, grouped, stream);
    else if (a.M <= 64) launch_skinny_mt<4>(a, blocks, grouped, stream);
    else return BITLINEAR_EUNSUPPORTED;
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_skinny(const Problem& p, int64_t M, void* ws, hipStream_t stream) {
    SkinnyArgs a{};
    a.p = p;
    a.M = (int32_t)M;
    const int64_t Kb = p.Kb;
    const int S = skinny_split_slices(M, p.N, p.K);
    a.sk.kb_per_slice = (int32_t)(ceil_div(ceil_div(Kb, S), 4) * 4);   // whole K-steps per slice
    a.sk.S = (int)ceil_div(Kb, a.sk.kb_per_slice);
    a.sk.partial = a.sk.S > 1 ? (int32_t*)ws : nullptr;
    a.nunits = ceil_div(p.N, kSkinnyRows) * a.sk.S;
    int rc = launch_skinny_any(a, false, stream);
    if (rc) return rc;
    if (a.sk.S > 1) return launch_splitk_epilogue(a.sk.partial, a.sk.S, M, p, stream);
    return BITLINEAR_OK;
}

// Grouped split-K epilogue (shared with the grouped prefill tiles, whose
// column tiles are 256 wide too), grid (units, row chunks): the workgroups
// of a block's first slice add the block's slices for kEpiRows token rows
// (thread = output row n of the block) and apply the dequant; every other
// unit, and blocks of unsplit problems, exit.  The slice loop is unrolled in
// rounds of kSkinnyMaxSlices, so that a thread's loads of a round are all in
// flight at once rather than one memory round trip per slice.
constexpr int kEpiRows = 4;

template <int W>   // unit width: output rows of a unit = threads of a workgroup
__global__ __launch_bounds__(W) void grouped_splitk_epilogue_kernel(const Problem* __restrict__ problems,
                                                                    const Unit* __restrict__ units, int64_t M,
                                                                    const int32_t* __restrict__ gpart) {
    const int64_t u = blockIdx.x;
    const Unit un = units[u];
    const Problem p = problems[un.problem];
    if (p.slices <= 1 || u - p.unit_begin != (int64_t)un.group * p.slices) return;
    const int64_t n = (int64_t)un.group * W + threadIdx.x;
    const int64_t m0 = (int64_t)blockIdx.y * kEpiRows;
    if (n >= p.N || m0 >= M) return;
    const int rows = M - m0 < kEpiRows ? (int)(M - m0) : kEpiRows;
    const int S = p.slices;
    const int32_t* __restrict__ src = gpart + (u * M + m0) * W + threadIdx.x;
    // The rows' scales, loaded together with the partial sums (rows past M
    // read row m0 and are never stored).
    float sc[kEpiRows];
#pragma unroll
    for (int r = 0; r < kEpiRows; ++r) sc[r] = dequant_scale(p.eta[m0 + (r < rows ? r : 0)], p.gamma);
    int v[kEpiRows] = {};
    if (S <= kSkinnyMaxSlices) {
        // every slice's loads in flight at once (straight-line code)
        int part[kSkinnyMaxSlices][kEpiRows];
#pragma unroll
        for (int s = 0; s < kSkinnyMaxSlices; ++s)
#pragma unroll
            for (int r = 0; r < kEpiRows; ++r)
                part[s][r] = s < S && r < rows ? src[((int64_t)s * M + r) * W] : 0;
#pragma unroll
        for (int r = 0; r < kEpiRows; ++r)
#pragma unroll
            for (int s = 0; s < kSkinnyMaxSlices; ++s) v[r] += part[s][r];
    } else {
        // more slices (base-3 plans of many tokens): rounds of
        // kSkinnyMaxSlices; the int32 sum is exact in any order
        for (int s0 = 0; s0 < S; s0 += kSkinnyMaxSlices) {
            int part[kSkinnyMaxSlices][kEpiRows];
#pragma unroll
            for (int s = 0; s < kSkinnyMaxSlices; ++s)
#pragma unroll
                for (int r = 0; r < kEpiRows; ++r)
                    part[s][r] = s0 + s < S && r < rows ? src[((int64_t)(s0 + s) * M + r) * W] : 0;
#pragma unroll
            for (int r = 0; r < kEpiRows; ++r)
#pragma unroll
                for (int s = 0; s < kSkinnyMaxSlices; ++s) v[r] += part[s][r];
        }
    }
#pragma unroll
    for (int r = 0; r < kEpiRows; ++r) {
        if (r >= rows) break;
        const int64_t m = m0 + r;
        p.y[m * p.N + n] = dequant(v[r], sc[r]);
        if (p.y_int) p.y_int[m * p.N + n] = v[r];
    }
}

int launch_skinny_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                          int32_t* partial, hipStream_t stream) {
    SkinnyArgs a{};
    a.problems = problems;
    a.units = units;
    a.gpart = partial;
    a.nunits = nunits;
    a.M = (int32_t)M;
    const int rc = launch_skinny_any(a, true, stream);
    if (rc || !partial) return rc;
    return launch_grouped_splitk_epilogue(problems, units, nunits, M, kSkinnyRows, partial, stream);
}

int launch_grouped_splitk_epilogue(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                                   int width, const int32_t* partial, hipStream_t stream) {
    const dim3 grid((unsigned)nunits, (unsigned)ceil_div(M, kEpiRows));
    if (width == 64)
        hipLaunchKernelGGL(grouped_splitk_epilogue_kernel<64>, grid, dim3(64), 0, stream, problems, units, M, partial);
    else if (width == 256)
        hipLaunchKernelGGL(grouped_splitk_epilogue_kernel<256>, grid, dim3(256), 0, stream, problems, units, M, partial);
    else
        return BITLINEAR_EINVAL;
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

}  // namespace bl
