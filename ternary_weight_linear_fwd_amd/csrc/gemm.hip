// gemm.hip -- prefill ternary x int8 contraction on the gfx950 matrix cores (M > 64).
//
// Where many tokens share the weights (prefill, batched decode) the
// contraction of [P2] "3. Additive Integer Accumulation" is a dense integer
// product, so it runs on v_mfma_i32_16x16x64_i8 with int32 accumulation
// (exact: |y_int| <= 127 * K < 2^31).
//
// Tiling.  A workgroup of WM x WN wavefronts computes a (WM*16*MT) x (WN*64)
// output tile; each wavefront owns MT x 4 MFMA tiles of 16 x 16.  The K loop
// advances 256 (four 64-k blocks) per step:
//  * A (activations, int8): the workgroup copies its rows x 256 bytes into LDS
//    with a 272-byte row stride (16-byte pad: the 16 rows a ds_read_b128
//    serves fall in distinct banks).
//  * B (weights): lane (n, g) of a wavefront loads the 16-byte chunk of row n
//    for k-block kb + g straight from the packed layout (four 256-byte runs
//    per wave load) and expands each 32-bit word into 16 ternary bytes in
//    VGPRs (shift, mask, one byte-permute per 4 weights); no LDS for B.
//  * Word d of that chunk feeds MFMA number d of the step for lane group g,
//    so the four MFMAs of a step together cover the 256 k exactly once; A is
//    read in the same (g, d) order.  The order of k inside a reduction is
//    free, so only the A/B agreement matters.
// Epilogue: y = float(acc) * ((eta[m] * gamma) / 127), fused.
#include "kernels.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kLdsRowBytes = 272;  // 256 data bytes + 16 pad

struct GemmArgs {
    Problem p;                // single mode
    const Problem* problems;  // grouped mode
    const Unit* units;        // grouped: (problem, column tile)
    int64_t M;
    int64_t ntiles_n;         // single: column tiles
    int64_t ntiles_m;         // single: row tiles
};

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8), each with its own L2.  Give each XCD a contiguous run of tiles
// (column index fastest) so that its L2 serves a few A row blocks to all of
// them and each B tile to the row blocks that run at the same time.
__device__ inline int64_t xcd_tile(int64_t b, int64_t T) {
    constexpr int64_t X = 8;
    const int64_t xcd = b % X, slot = b / X, q = T / X, r = T % X;
    return xcd * q + (xcd < r ? xcd : r) + slot;
}

// ---------------------------------------------------------------------------
// Prefill variant (M > 64): 128 x 256 workgroup tile, four wavefronts side by
// side in N; each owns all 128 rows x 64 columns as 4 x 2 tiles of
// v_mfma_i32_32x32x32_i8, so every weight word is expanded exactly once per
// workgroup.  The K loop advances 128 (two 64-k blocks) per step and keeps
// three steps in flight ahead of the one being computed:
//  * A: a four-stage LDS ring of 128 rows x 128 bytes, filled by direct
//    global->LDS loads (global_load_lds_dwordx4, 1 KB per wave instruction).
//    Chunk c (16 bytes) of row r is stored at chunk c ^ ((r >> 1) & 7): the 16
//    rows one ds_read_b128 phase serves land on 16 distinct bank groups, with
//    no padding, so each wave's 1 KB DMA stays contiguous.
//  * B: the packed words go straight to registers (a four-slot ring); each
//    lane expands them into ternary bytes right before the MFMAs that use
//    them.  Lane (n, g) holds row n's k-block kb + g; word d feeds MFMA group
//    d, whose 32 k are the two lane groups' 16-k runs; A is read in the same
//    (g, d) order.
// Rows past M and k past K are read from clamped (in-bounds) addresses: rows
// past M are never stored, and every k past K meets a zero weight (pad code
// 01 inside the last block, code 01 forced for blocks past the end).
constexpr int kPreBN = 256;
constexpr int kPreStages = 4;

typedef int v16i __attribute__((ext_vector_type(16)));

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector memory
// operations are outstanding; expcnt and lgkmcnt are left unconstrained.
template <int vm>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(vm >= 0 && vm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14));
}

// One 16-byte-per-lane direct global->LDS load (the wave's 64 lanes fill
// 1 KB at lds_dst).  Kept as a plain (non-template) function: the host
// compilation pass rejects template instantiations that name this builtin.
__device__ __forceinline__ void dma_16(const void* src, void* lds_dst) {
    __builtin_amdgcn_global_load_lds(src, lds_dst, 16, 0, 0);
}

template <int MT>
struct PrefillCtx {
    static constexpr int BM = 32 * MT;            // rows per workgroup tile
    static constexpr int AStage = BM * 128;       // bytes of one A stage
    static constexpr int NA = AStage / 4096;      // A DMA instructions per wave per step
    uint8_t* lds;
    const int8_t* asrc[NA];
    int acol[NA];
    const uint4* brow;
    int64_t K, Kb, nsteps;
    int wave, lane, ln, lg;
};

// Queue step `step`: this wave's NA 1 KB A DMAs into LDS stage `stage` and
// this lane's two B chunks into registers: NA + 2 vector memory instructions.
template <int MT>
__device__ __forceinline__ void prefill_issue(const PrefillCtx<MT>& c, int stage, uint4 (&bq)[2],
                                              int64_t step) {
    uint8_t* st = c.lds + stage * PrefillCtx<MT>::AStage;
    const int64_t kbase = step * 128;
    const bool full = kbase + 128 <= c.K;
#pragma unroll
    for (int j = 0; j < PrefillCtx<MT>::NA; ++j) {
        const int8_t* src = c.asrc[j] + kbase;
        if (!full && kbase + c.acol[j] >= c.K) src = c.asrc[j] + (c.K - 16 - c.acol[j]);
        dma_16(src, st + (j * 4 + c.wave) * 1024);
    }
    int64_t kb = step * 2 + c.lg;
    kb = kb < c.Kb ? kb : c.Kb - 1;   // a block past the end is zeroed at use
#pragma unroll
    for (int t = 0; t < 2; ++t) bq[t] = c.brow[kb * 64 + t * 32];
}

// One K-step of MFMAs from LDS stage `stage` and the B words `bq`.
template <int MT>
__device__ __forceinline__ void prefill_compute(const PrefillCtx<MT>& c, int stage, const uint4 (&bq)[2],
                                                int64_t step, v16i (&acc)[MT][2]) {
    const uint8_t* A = c.lds + stage * PrefillCtx<MT>::AStage;
    const bool kb_ok = step * 2 + c.lg < c.Kb;
    uint4 bw[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        bw[t] = kb_ok ? bq[t] : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
    // Two register sets for the A fragments and the expanded B words: group
    // d+1's LDS reads and expansion run while group d's eight MFMAs execute.
    v4i af[2][MT], bf[2][2];
    auto load_a = [&](v4i (&dst)[MT], int d) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const int r = i * 32 + c.ln;
            dst[i] = *reinterpret_cast<const v4i*>(A + r * 128 + (((c.lg * 4 + d) ^ ((r >> 1) & 7)) << 4));
        }
    };
    auto expand_b = [&](v4i (&dst)[2], int d) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t w = d == 0 ? bw[t].x : d == 1 ? bw[t].y : d == 2 ? bw[t].z : bw[t].w;
            dst[t].x = (int)codes_to_ternary(w & 0x03030303u);
            dst[t].y = (int)codes_to_ternary((w >> 2) & 0x03030303u);
            dst[t].z = (int)codes_to_ternary((w >> 4) & 0x03030303u);
            dst[t].w = (int)codes_to_ternary((w >> 6) & 0x03030303u);
        }
    };
    load_a(af[0], 0);
    expand_b(bf[0], 0);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int cur = d & 1;
        if (d < 3) load_a(af[cur ^ 1], d + 1);
        __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of this group's MFMAs
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < MT; ++i)
                acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bf[cur][t], acc[i][t], 0, 0, 0);
        if (d < 3) expand_b(bf[cur ^ 1], d + 1);
    }
}

// Step `step` of the ring: wait for its data (exactly: the steps issued after
// it may stay in flight), make that true for every wave, refill the stage
// freed by step-1 with step+3, compute.  Every LDS read of that stage fed an
// MFMA before the barrier.  A plain s_barrier: __syncthreads() would also
// drain the DMAs still in flight.
template <int MT>
__device__ __forceinline__ void prefill_step(const PrefillCtx<MT>& c, int stage, const uint4 (&bcur)[2],
                                             uint4 (&bnext)[2], int64_t step, v16i (&acc)[MT][2]) {
    constexpr int ops = PrefillCtx<MT>::NA + 2;   // vector memory instructions per step
    if (step >= c.nsteps) return;
    if (step + 2 < c.nsteps) wait_vmcnt<2 * ops>();
    else if (step + 1 < c.nsteps) wait_vmcnt<ops>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (step + 3 < c.nsteps) prefill_issue<MT>(c, (stage + 3) & 3, bnext, step + 3);
    prefill_compute<MT>(c, stage, bcur, step, acc);
}

template <int MT, bool GROUPED>
__global__ __launch_bounds__(256, 2) void gemm_prefill_kernel(GemmArgs a) {
    using Ctx = PrefillCtx<MT>;
    constexpr int kPreBM = Ctx::BM;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kPreStages * Ctx::AStage];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    Problem p;
    int64_t tile_n, tile_m;
    if constexpr (GROUPED) {
        const Unit un = a.units[blockIdx.x];
        p = a.problems[un.problem];
        tile_n = un.group;
        tile_m = blockIdx.y;
    } else {
        p = a.p;
        const int64_t tile = xcd_tile(blockIdx.x, a.ntiles_n * a.ntiles_m);
        tile_m = tile / a.ntiles_n;
        tile_n = tile - tile_m * a.ntiles_n;
    }
    const int64_t M = a.M, N = p.N, K = p.K, Kb = p.Kb;
    const int64_t m0 = tile_m * kPreBM;
    const int64_t group = tile_n * 4 + wave;
    const bool group_ok = group < ceil_div(N, 64);

    Ctx c;
    c.lds = lds;
    c.K = K;
    c.Kb = Kb;
    c.nsteps = ceil_div(Kb, 2);
    c.wave = wave;
    c.lane = lane;
    c.ln = lane & 31;
    c.lg = lane >> 5;
#pragma unroll
    for (int j = 0; j < Ctx::NA; ++j) {
        const int P = (j * 4 + wave) * 64 + lane;       // physical 16-byte slot
        const int r = P >> 3;
        c.acol[j] = ((P & 7) ^ ((r >> 1) & 7)) * 16;    // logical byte column
        const int64_t m = m0 + r < M ? m0 + r : M - 1;
        c.asrc[j] = p.xq + m * K + c.acol[j];
    }
    c.brow = p.packed + (group_ok ? group : 0) * Kb * 64 + c.ln;

    v16i acc[MT][2];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][t][e] = 0;

    uint4 b0[2], b1[2], b2[2], b3[2];
    if (0 < c.nsteps) prefill_issue<MT>(c, 0, b0, 0);
    if (1 < c.nsteps) prefill_issue<MT>(c, 1, b1, 1);
    if (2 < c.nsteps) prefill_issue<MT>(c, 2, b2, 2);
    for (int64_t s = 0; s < c.nsteps; s += 4) {
        prefill_step<MT>(c, 0, b0, b3, s + 0, acc);
        prefill_step<MT>(c, 1, b1, b0, s + 1, acc);
        prefill_step<MT>(c, 2, b2, b1, s + 2, acc);
        prefill_step<MT>(c, 3, b3, b2, s + 3, acc);
    }

    // Epilogue: element 4j + q of tile (i, t) is row 32i + 8j + 4lg + q, column 32t + ln.
    if (!group_ok) return;
    const int ln = c.ln, lg = c.lg;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t m = m0 + i * 32 + j * 8 + lg * 4 + q;
                if (m >= M) continue;
                const float sc = dequant_scale(p.eta[m], p.gamma);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int64_t n = group * 64 + t * 32 + ln;
                    if (n >= N) continue;
                    const int v = acc[i][t][j * 4 + q];
                    p.y[m * N + n] = dequant(v, sc);
                    if (p.y_int) p.y_int[m * N + n] = v;
                }
            }
        }
    }
}

// Column tile width (output rows of W per workgroup) of the prefill kernel.
static int gemm_bn(int64_t M) { (void)M; return kPreBN; }

// Prefill tile height.  64-row tiles (158 VGPRs, 32 KB LDS: three workgroups
// per CU, 768 slots on 256 CUs) balance far better at prefill sizes such as
// M = 2048; 128-row tiles (two per CU) reuse each expanded weight word twice
// as often and only pay off once the grid is many rounds deep.
static int prefill_mt(int64_t M, int64_t N) {
    const int64_t t64 = ceil_div(M, 64) * ceil_div(N, kPreBN);
    return t64 <= 4 * 768 ? 2 : 4;
}

static int dispatch(GemmArgs& a, int64_t ntn, bool grouped, hipStream_t stream) {
    const int64_t M = a.M;
    if (grouped) {   // grouped prefill keeps 128-row tiles (grid.y = row tiles)
        hipLaunchKernelGGL((gemm_prefill_kernel<4, true>), dim3((unsigned)ntn, (unsigned)ceil_div(M, 128)),
                           dim3(256), 0, stream, a);
    } else {
        const int mt = prefill_mt(M, a.p.N);
        a.ntiles_n = ntn;
        a.ntiles_m = ceil_div(M, 32 * mt);
        if (mt == 2)
            hipLaunchKernelGGL((gemm_prefill_kernel<2, false>), dim3((unsigned)(ntn * a.ntiles_m)),
                               dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((gemm_prefill_kernel<4, false>), dim3((unsigned)(ntn * a.ntiles_m)),
                               dim3(256), 0, stream, a);
    }
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int launch_gemm(const Problem& p, int64_t M, hipStream_t stream) {
    GemmArgs a{};
    a.p = p;
    a.M = M;
    const int64_t ntn = ceil_div(p.N, gemm_bn(M));
    return dispatch(a, ntn, false, stream);
}

int gemm_tile_n(int64_t M) { return gemm_bn(M); }

int launch_gemm_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                        hipStream_t stream) {
    GemmArgs a{};
    a.problems = problems;
    a.units = units;
    a.M = M;
    return dispatch(a, nunits, true, stream);
}

}  // namespace bl
