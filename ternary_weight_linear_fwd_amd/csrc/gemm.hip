// gemm.hip -- prefill ternary x int8 contraction on the gfx950 matrix cores (M > 64).
//
// Where many tokens share the weights (prefill, batched decode) the
// contraction of [P2] "3. Additive Integer Accumulation" is a dense integer
// product; it runs on v_mfma_i32_32x32x32_i8 with int32 accumulation.
//
// Workgroup tile: BM = 32*MT token rows x 128*NT weight rows (output
// columns), MT x NT in {2 x 2, 3 x 3, 4 x 2}, chosen per shape.  Four
// wavefronts sit side by side in N; each owns all BM rows x 32*NT columns as
// MT x NT MFMA tiles of 32 x 32, so every packed weight word is expanded
// once per workgroup.  The K loop advances 128 (two 64-k blocks) per step
// through a ring of three stages (four for 128-row tiles), keeping the next
// steps in flight while one is computed.  The kernel tracks the completion
// of its own loads: an explicit vmcnt wait and one barrier per step.
//  * A (int8 activations) arrives by direct global->LDS loads
//    (global_load_lds_dwordx4, 1 KB per wave instruction): BM rows x 128
//    bytes per stage.  Chunk c (16 bytes) of row r is stored at chunk
//    c ^ ((r >> 1) & 7): the 16 rows one ds_read_b128 phase serves land on
//    distinct banks, and each wave's 1 KB DMA stays contiguous.
//  * B (packed codes) is private to each wavefront, so it goes straight to
//    registers (one 16-byte load per lane and column tile per step, a ring
//    of register sets matching the LDS stages) and is expanded there.
// Lane (n, g) reads row n's 16-byte chunk of k-block 2*step + g; word d of it
// feeds MFMA group d, whose 32 k are the two lane groups' 16-k runs, and A is
// read in the same (g, d) order (the order of k inside a reduction is free;
// only the A/B agreement matters).
//
// The codes go to the MFMA as they are: with c = w + 1 in {0, 1, 2} (field j
// of a word is (w >> 2j) & 0x03030303),
//     sum_k x_k w_k = sum_k x_k c_k - sum_k x_k .
// The row sums sum_k x_k are either given (the activation quantizer writes
// them; every k at or past K then gets code 00, so it adds nothing) or taken
// from the same LDS fragments (v_dot4 against ones; wavefront w sums word
// group w of every step), in which case every k whose code is 01 -- pads
// inside the last block, blocks past the end (forced to 01), and k past K
// read from clamped addresses -- contributes equally to both terms and
// cancels.  Raw codes also toggle far fewer multiplier bits than -1/0/+1
// bytes, which lets the matrix cores hold a higher clock.  int32 arithmetic
// wraps, so the difference is exact whenever the result fits
// (|y_int| <= 127 K < 2^31).
// Epilogue: y = float(y_int) * ((eta[m] * gamma) / 127), fused.
#include <atomic>

#include "gemm.hpp"
#include "kernels.hpp"
#include "xcd.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct GemmArgs {
    Problem p;                // single mode
    const Problem* problems;  // grouped mode
    const Unit* units;        // grouped: (problem, column tile)
    int64_t M;
    int64_t ntiles_n;         // single: column tiles
    int64_t ntiles_m;         // single: row tiles
    const int32_t* xsum;      // single: the row sums sum_k xq[m][k], or null
    int32_t* partial;         // single, split K: [S][M][N] int32 partial sums, or null
    int32_t S;                // single: K-slices per tile (1: no split)
    int32_t sps;              // single, split K: 128-k steps per slice
};

// Tile order: each XCD takes a contiguous run of the tile order
// (xcd_contiguous), and the order walks the grid in bands of `band` row
// tiles, row index fastest inside a band, so the tiles an XCD runs at one time
// cover a compact block (about 10 x 10 tiles of 64 x 256): its L2 then serves
// their activation rows and weight columns to all of them.
// Tile counts stay below 2^26 (M * N < 2^40), so 32-bit arithmetic suffices.
__device__ inline void tile_coords(uint32_t b, uint32_t ntm, uint32_t ntn, uint32_t band, int64_t& tm,
                                   int64_t& tn) {
    const uint32_t t = xcd_contiguous(b, ntm * ntn);
    const uint32_t bi = t / (band * ntn);
    const uint32_t rows = ntm - bi * band < band ? ntm - bi * band : band;
    const uint32_t within = t - bi * band * ntn;
    tm = bi * band + within % rows;
    tn = within / rows;
}

constexpr int kPreBN = 256;

// s_waitcnt immediate (gfx9 encoding): wait until at most `vm` vector memory
// operations are outstanding; expcnt and lgkmcnt are left unconstrained.
template <int vm>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(vm >= 0 && vm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((vm & 15) | (7 << 4) | (15 << 8) | ((vm >> 4) << 14));
}

// One 16-byte-per-lane direct global->LDS load (the wave's 64 lanes fill
// 1 KB at lds_dst).  This builtin keeps the LDS destination as a typed
// address, so the compiler knows which LDS object the load writes and does
// not make reads of the other stages wait for it.  Kept as a plain
// (non-template) function: the host compilation pass rejects template
// instantiations that name it.
__device__ __forceinline__ void dma_16(const void* src, void* lds_dst) {
    __builtin_amdgcn_load_to_lds(const_cast<void*>(src),
                                 (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

template <int MT, int NT>
struct PrefillCtx {
    static constexpr int BM = 32 * MT;            // token rows per workgroup tile
    static constexpr int AStage = BM * 128;       // bytes of A per stage
    static constexpr int NA = AStage / 4096;      // A DMA instructions per wave per step
    // Vector memory instructions per step: NA activation DMAs, plus NT weight
    // loads for a wavefront with columns inside N.
    static constexpr int ops(bool act) { return NA + (act ? NT : 0); }
    // DMA sources are a wave-uniform base (scalar registers) plus a 32-bit
    // per-lane offset, so that the main loop spends no vector ALU work on
    // addresses (row offsets stay below 2^32: 128 rows x K <= 2^21).
    const int8_t* abase;    // the tile's first activation row
    uint32_t aoff[NA];      // (row in the tile, clamped below M) * K + byte column
    uint32_t acol[NA];      // byte column inside the 128-k step
    const uint8_t* bbase[NT];   // k-block 0 of the 32 weight rows of the wavefront's column tile t
    uint32_t boff;              // lane (ln, lg): row ln's 16 bytes of k-block lg of a step
    uint32_t afrag[4];      // LDS offset of this lane's A fragment of group d, row tile 0
    uint32_t sxfrag;        // afrag[wave]: the word group this wavefront sums
    int64_t K, Kb, nsteps;
    int64_t kstep0;         // first step of this workgroup's K-slice (steps count from it)
    int wave, lane, ln, lg;
};

// Queue step `step`: this wave's NA activation DMAs into LDS stage `st` and
// its NT weight loads into registers bq (the weight chunks are private to
// the wavefront, so they skip LDS).  CHECKED: the step may reach past K (the
// last step, or one queued past the end), so addresses are clamped in
// bounds; otherwise all 128 k of the step lie inside K.  ACT false: the
// wavefront has no columns inside N and loads only its share of A.
template <int MT, int NT, bool CHECKED, bool ACT>
__device__ __forceinline__ void prefill_issue(const PrefillCtx<MT, NT>& c, uint8_t* st, int64_t step, v4i (&bq)[NT]) {
    using Ctx = PrefillCtx<MT, NT>;
    if constexpr (NT == 3) __builtin_amdgcn_sched_barrier(0);
    const int64_t as = c.kstep0 + step;   // step in the whole K loop
    const int64_t kbase = as * 128;
#pragma unroll
    for (int j = 0; j < Ctx::NA; ++j) {
        const int8_t* src;
        if constexpr (CHECKED) {
            const uint32_t o = kbase + c.acol[j] >= c.K ? c.aoff[j] - c.acol[j] + (uint32_t)(c.K - 16)
                                                        : c.aoff[j] + (uint32_t)kbase;
            src = c.abase + o;
        } else {
            src = (c.abase + kbase) + c.aoff[j];
        }
        dma_16(src, st + (j * 4 + c.wave) * 1024);
    }
    // Lane (ln, lg) takes row ln of each column tile's 32 rows in k-block
    // 2 * step + lg.
#pragma unroll
    for (int t = 0; t < (ACT ? NT : 0); ++t) {
        const uint8_t* bsrc;
        if constexpr (CHECKED) {
            const int64_t kb = as * 2 + c.lg < c.Kb ? as * 2 + c.lg : c.Kb - 1;   // past the end: replaced at use
            bsrc = c.bbase[t] + (uint32_t)(kb * 1024 + (c.boff & 1023u));
        } else {
            bsrc = (c.bbase[t] + as * 2048) + c.boff;
        }
        bq[t] = *reinterpret_cast<const v4i*>(bsrc);
    }
    // The explicit vmcnt waits count on each step's loads being issued as one
    // group, in step order.  Under the register pressure of the 96 x 384 tile
    // the scheduler otherwise interleaves the groups (and then waits for
    // everything); the other tiles keep them in order by themselves and run
    // faster without the fence.
    if constexpr (NT == 3) __builtin_amdgcn_sched_barrier(0);
}

// One K-step of MFMAs from the LDS stage at A.  Without given row sums (RS
// false) wavefront w also adds word group w of the step's A rows into the row
// sums `sx` (one extra fragment read per row tile, four v_dot4 each).  TAIL:
// the step may be the last one, whose second k-block can lie past the end.
// ACT false: no columns inside N, so only the row sums (if any).
template <int MT, int NT, bool TAIL, bool RS, bool ACT>
__device__ __forceinline__ void prefill_compute(const PrefillCtx<MT, NT>& c, const uint8_t* A, int64_t step,
                                                const v4i (&bq)[NT], v16i (&acc)[MT][NT], int (&sx)[MT]) {
    v4i bw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) bw[t] = bq[t];
    if constexpr (TAIL) {
        const int64_t as = c.kstep0 + step;   // step in the whole K loop
        if constexpr (RS) {
            // The given row sums cover k < K only, so every k at or past K
            // gets code 00 (c = 0): it adds nothing whatever A holds there.
            // Word d of the lane's chunk is k = 64 kb + 16 d .. + 15, and K
            // is a multiple of 16, so a word is wholly inside or outside.
            const int64_t k0 = (as * 2 + c.lg) * 64;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                if (k0 + 16 * d >= c.K) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) bw[t][d] = 0;
                }
        } else if (as * 2 + 1 >= c.Kb && c.lg == 1) {   // k-block past the end: code 01
#pragma unroll
            for (int t = 0; t < NT; ++t) bw[t] = v4i{0x55555555, 0x55555555, 0x55555555, 0x55555555};
        }
    }
    // Row 32i + ln, chunk ((lg & 1) * 4 + d) ^ ((row >> 1) & 7): the swizzle
    // term is the same for every row tile i, so the per-lane offsets are
    // computed once and i enters as an immediate offset.  The masks bound
    // every LDS offset visibly, so that the compiler can prove each read stays
    // inside this stage's object and tell it apart from the loads in flight
    // into the other stages.
    auto a_frag = [&](int i, int d) {
        return *reinterpret_cast<const v4i*>(A + i * 4096 + (c.afrag[d & 3] & 4095u));
    };
    if constexpr (!RS) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            const v4i f = *reinterpret_cast<const v4i*>(A + i * 4096 + (c.sxfrag & 4095u));
            sx[i] = __builtin_amdgcn_sdot4(f.x, 0x01010101, sx[i], false);
            sx[i] = __builtin_amdgcn_sdot4(f.y, 0x01010101, sx[i], false);
            sx[i] = __builtin_amdgcn_sdot4(f.z, 0x01010101, sx[i], false);
            sx[i] = __builtin_amdgcn_sdot4(f.w, 0x01010101, sx[i], false);
        }
    }
    if constexpr (!ACT) return;
    // Two register sets for the A fragments and the B codes: group d+1's LDS
    // reads and field extraction run while group d's MFMAs execute.
    v4i af[2][MT], bf[2][NT];
    auto load_a = [&](v4i (&dst)[MT], int d) {
#pragma unroll
        for (int i = 0; i < MT; ++i) dst[i] = a_frag(i, d);
    };
    auto fields = [&](v4i (&dst)[NT], int d) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint32_t w = (uint32_t)bw[t][d];
            dst[t].x = (int)(w & 0x03030303u);
            dst[t].y = (int)((w >> 2) & 0x03030303u);
            dst[t].z = (int)((w >> 4) & 0x03030303u);
            dst[t].w = (int)((w >> 6) & 0x03030303u);
        }
    };
    load_a(af[0], 0);
    if constexpr (MT * NT <= 4) fields(bf[0], 0);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int cur = d & 1;
        if (d < 3) load_a(af[cur ^ 1], d + 1);
        __builtin_amdgcn_sched_barrier(0);   // keep those reads ahead of this group's MFMAs
        if constexpr (MT * NT <= 4) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], bf[cur][t], acc[i][t], 0, 0, 0);
            if (d < 3) fields(bf[cur ^ 1], d + 1);
        } else {
            // Wide tiles: one set of expanded codes (register budget); each
            // weight word's fields are taken just before their MT MFMAs.
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint32_t w = (uint32_t)bw[t][d];
                const v4i f = v4i{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                                  (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cur][i], f, acc[i][t], 0, 0, 0);
            }
        }
    }
}

// A step of a ring of NS stages that is not among the last ones: wait until
// its data has landed (the next NS - 2 steps' loads stay in flight), make
// that true for every wave, refill the stage that step - 1 read (every wave
// is past it) with step + NS - 1, compute.  Straight-line code, so that the
// compiler can see which stage each LDS read and each load in flight touch
// and adds no waits of its own.
template <int MT, int NT, int NS, bool RS, bool ACT>
__device__ __forceinline__ void prefill_step(const PrefillCtx<MT, NT>& c, const uint8_t* cur, uint8_t* refill,
                                             int64_t step, const v4i (&bq_cur)[NT], v4i (&bq_refill)[NT],
                                             v16i (&acc)[MT][NT], int (&sx)[MT]) {
    wait_vmcnt<(NS - 2) * PrefillCtx<MT, NT>::ops(ACT)>();
    __builtin_amdgcn_s_barrier();   // not __syncthreads(): that would drain the loads in flight
    prefill_issue<MT, NT, false, ACT>(c, refill, step + NS - 1, bq_refill);   // <= nsteps - 2: never the last
    prefill_compute<MT, NT, false, RS, ACT>(c, cur, step, bq_cur, acc, sx);
}

// Any step, including the last ones (nothing left to refill, or past the end).
template <int MT, int NT, int NS, bool RS, bool ACT>
__device__ __forceinline__ void prefill_step_tail(const PrefillCtx<MT, NT>& c, const uint8_t* cur, uint8_t* refill,
                                                  int64_t step, const v4i (&bq_cur)[NT], v4i (&bq_refill)[NT],
                                                  v16i (&acc)[MT][NT], int (&sx)[MT]) {
    constexpr int Ops = PrefillCtx<MT, NT>::ops(ACT);
    if (step >= c.nsteps) return;
    const int64_t later = c.nsteps - 1 - step;   // queued steps after this one
    if (NS >= 4 && later >= 2) wait_vmcnt<(NS >= 4 ? 2 : 1) * Ops>();
    else if (later >= 1) wait_vmcnt<Ops>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (step + NS - 1 < c.nsteps) prefill_issue<MT, NT, true, ACT>(c, refill, step + NS - 1, bq_refill);
    prefill_compute<MT, NT, true, RS, ACT>(c, cur, step, bq_cur, acc, sx);
}

// The K loop over a ring of NS LDS stages (each its own LDS object, so that
// the compiler can tell a read of one stage from the loads in flight into
// the others).
template <int MT, int NT, int NS, bool RS, bool ACT>
__device__ __forceinline__ void prefill_pipeline(const PrefillCtx<MT, NT>& c, uint8_t* stage0, uint8_t* stage1,
                                                 uint8_t* stage2, uint8_t* stage3, v16i (&acc)[MT][NT],
                                                 int (&sx)[MT]) {
    // The first NS - 1 steps are always queued (past the end they read clamped,
    // in-bounds addresses and are never used), so that no branch precedes the
    // main loop.  Weight words of the steps in flight: one register set per
    // stage.
    v4i bq0[NT], bq1[NT], bq2[NT], bq3[NT];
    prefill_issue<MT, NT, true, ACT>(c, stage0, 0, bq0);
    prefill_issue<MT, NT, true, ACT>(c, stage1, 1, bq1);
    if constexpr (NS == 4) prefill_issue<MT, NT, true, ACT>(c, stage2, 2, bq2);
    int64_t step = 0;
    if constexpr (NS == 3) {
        // The main loop queues steps up to nsteps - 2, all of them whole.
        for (; step + 6 <= c.nsteps; step += 3) {
            prefill_step<MT, NT, 3, RS, ACT>(c, stage0, stage2, step, bq0, bq2, acc, sx);
            prefill_step<MT, NT, 3, RS, ACT>(c, stage1, stage0, step + 1, bq1, bq0, acc, sx);
            prefill_step<MT, NT, 3, RS, ACT>(c, stage2, stage1, step + 2, bq2, bq1, acc, sx);
        }
        // The last one to five steps.
        prefill_step_tail<MT, NT, 3, RS, ACT>(c, stage0, stage2, step, bq0, bq2, acc, sx);
        prefill_step_tail<MT, NT, 3, RS, ACT>(c, stage1, stage0, step + 1, bq1, bq0, acc, sx);
        prefill_step_tail<MT, NT, 3, RS, ACT>(c, stage2, stage1, step + 2, bq2, bq1, acc, sx);
        prefill_step_tail<MT, NT, 3, RS, ACT>(c, stage0, stage2, step + 3, bq0, bq2, acc, sx);
        prefill_step_tail<MT, NT, 3, RS, ACT>(c, stage1, stage0, step + 4, bq1, bq0, acc, sx);
    } else {
        for (; step + 8 <= c.nsteps; step += 4) {
            prefill_step<MT, NT, 4, RS, ACT>(c, stage0, stage3, step, bq0, bq3, acc, sx);
            prefill_step<MT, NT, 4, RS, ACT>(c, stage1, stage0, step + 1, bq1, bq0, acc, sx);
            prefill_step<MT, NT, 4, RS, ACT>(c, stage2, stage1, step + 2, bq2, bq1, acc, sx);
            prefill_step<MT, NT, 4, RS, ACT>(c, stage3, stage2, step + 3, bq3, bq2, acc, sx);
        }
        // The last one to seven steps.
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage0, stage3, step, bq0, bq3, acc, sx);
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage1, stage0, step + 1, bq1, bq0, acc, sx);
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage2, stage1, step + 2, bq2, bq1, acc, sx);
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage3, stage2, step + 3, bq3, bq2, acc, sx);
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage0, stage3, step + 4, bq0, bq3, acc, sx);
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage1, stage0, step + 5, bq1, bq0, acc, sx);
        prefill_step_tail<MT, NT, 4, RS, ACT>(c, stage2, stage1, step + 6, bq2, bq1, acc, sx);
    }

}

// Resident workgroups per CU for an MT x NT wave tile (register budget).
constexpr int prefill_occupancy(int mt, int nt) { return mt * nt <= 2 ? 4 : mt * nt <= 4 ? 3 : 2; }

// RS: the row sums come from a.xsum (single mode) instead of being summed
// from the activation tiles on the way.
template <int MT, int NT, bool GROUPED, int NS, bool RS>
__global__ __launch_bounds__(256, prefill_occupancy(MT, NT)) void gemm_prefill_kernel(GemmArgs a) {
    static_assert(NS == 3 || NS == 4, "ring of three or four stages");
    using Ctx = PrefillCtx<MT, NT>;
    constexpr int BM = Ctx::BM;
    // K split: single launches of 32 x 128 tiles, grouped launches of
    // 64 x 256 tiles (the larger tiles have no registers to spare for it).
    constexpr bool SPLIT = (!GROUPED && MT == 1 && NT == 1) || (GROUPED && MT == 2 && NT == 2);
    // Up to four stages, each its own LDS object, so that the compiler can
    // tell a read of one stage from the loads in flight into the others.
    __shared__ __attribute__((aligned(1024))) uint8_t stage0[Ctx::AStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage1[Ctx::AStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage2[Ctx::AStage];
    __shared__ __attribute__((aligned(1024))) uint8_t stage3[NS == 4 ? Ctx::AStage : 16];
    __shared__ int rowsum_part[RS ? 1 : 8][BM];   // [wave * 2 + lane group][row]
    __shared__ float2 rowinfo[BM];   // (row sum as int bits, dequant scale)

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    Problem p;
    int64_t tile_n, tile_m, slice = 0;
    if constexpr (GROUPED) {
        const Unit un = a.units[blockIdx.x];
        p = a.problems[un.problem];
        tile_n = un.group;
        tile_m = blockIdx.y;
        // Split plans: the K-slices of a column tile are adjacent units.
        if (SPLIT && p.slices > 1) slice = (int64_t)blockIdx.x - p.unit_begin - tile_n * p.slices;
    } else {
        p = a.p;
        // Split K: consecutive workgroups are the slices of one tile.
        const uint32_t S = SPLIT && a.S > 1 ? (uint32_t)a.S : 1u;
        slice = SPLIT ? blockIdx.x % S : 0;
        tile_coords(SPLIT ? blockIdx.x / S : blockIdx.x, (uint32_t)a.ntiles_m, (uint32_t)a.ntiles_n, 16 / MT, tile_m,
                    tile_n);
    }
    const int64_t M = a.M, N = p.N, K = p.K, Kb = p.Kb;
    const int64_t m0 = tile_m * BM;
    // Column tile t of this wavefront: 32-column block cb0 + t, the rows
    // 32 * (cb & 1) .. + 31 of 64-row weight group cb / 2.
    const int64_t cb0 = tile_n * (4 * NT) + (int64_t)wave * NT;
    const bool group_ok = cb0 * 32 < N;   // any of the wavefront's columns inside N

    Ctx c;
    c.K = K;
    c.Kb = Kb;
    c.kstep0 = 0;
    c.nsteps = ceil_div(Kb, 2);
    const bool split = SPLIT && (GROUPED ? p.slices > 1 : a.S > 1);
    if (split) {   // this slice's steps (never empty: the host sizes slices)
        const int64_t sps = GROUPED ? ceil_div(c.nsteps, (int64_t)p.slices) : (int64_t)a.sps;
        c.kstep0 = slice * sps;
        c.nsteps = c.nsteps - c.kstep0 < sps ? c.nsteps - c.kstep0 : sps;
    }
    c.wave = wave;
    c.lane = lane;
    c.ln = lane & 31;
    c.lg = lane >> 5;
    c.abase = p.xq + m0 * K;
#pragma unroll
    for (int j = 0; j < Ctx::NA; ++j) {
        const int P = (j * 4 + wave) * 64 + lane;       // physical 16-byte slot
        const int r = P >> 3;
        c.acol[j] = (uint32_t)(((P & 7) ^ ((r >> 1) & 7)) * 16);   // logical byte column
        const int64_t rr = m0 + r < M ? r : M - 1 - m0;
        c.aoff[j] = (uint32_t)(rr * K) + c.acol[j];
    }
    const int64_t ngroups = ceil_div(N, 64);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t cb = cb0 + t, g = cb >> 1;
        c.bbase[t] = reinterpret_cast<const uint8_t*>(p.packed) + (g < ngroups ? g : 0) * Kb * 1024 + (cb & 1) * 512;
    }
    c.boff = (uint32_t)(c.lg * 1024 + c.ln * 16);
#pragma unroll
    for (int d = 0; d < 4; ++d)
        c.afrag[d] = (uint32_t)((c.ln & 31) * 128 + ((((c.lg & 1) * 4 + d) ^ ((c.ln >> 1) & 7)) << 4));
    c.sxfrag = (uint32_t)((c.ln & 31) * 128 + ((((c.lg & 1) * 4 + (wave & 3)) ^ ((c.ln >> 1) & 7)) << 4));

    v16i acc[MT][NT];
    int sx[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        sx[i] = 0;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][t][e] = 0;
    }

    // Wavefronts with no columns inside N (the last column tile of a ragged
    // N) only keep the shared activation ring moving.
    if (group_ok) prefill_pipeline<MT, NT, NS, RS, true>(c, stage0, stage1, stage2, stage3, acc, sx);
    else prefill_pipeline<MT, NT, NS, RS, false>(c, stage0, stage1, stage2, stage3, acc, sx);

    // Row sums: partials of (wave, lane group) -> one total per tile row, and
    // each row's dequant scale, computed once here rather than by every lane
    // that stores a value of the row.
    if constexpr (!RS) {
#pragma unroll
        for (int i = 0; i < MT; ++i) rowsum_part[wave * 2 + c.lg][i * 32 + c.ln] = sx[i];
        __syncthreads();
    }
    if (tid < BM) {
        const int64_t m = m0 + tid;
        int t = 0;
        if constexpr (RS) {
            // Under split K the whole row sum is taken off once, by slice 0.
            t = m < M && (!SPLIT || slice == 0) ? a.xsum[m] : 0;
        } else {
#pragma unroll
            for (int w = 0; w < 8; ++w) t += rowsum_part[w][tid];
        }
        rowinfo[tid] = make_float2(__int_as_float(t), m < M ? dequant_scale(p.eta[m], p.gamma) : 0.0f);
    }
    __syncthreads();

    // Epilogue: element 4j + q of tile (i, t) is row 32i + 8j + 4lg + q, column 32t + ln.
    if (!group_ok) return;
    const int ln = c.ln, lg = c.lg;
    const int64_t n0 = cb0 * 32 + ln;
    bool col[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) col[t] = n0 + 32 * t < N;
    if (split) {
        // Split K: this slice's integer sums (its own row sums taken off);
        // the split-K epilogue adds the slices in order and dequantizes.
        // Single: [S][M][N]; grouped: [unit][M][256].
        int32_t* pcol = GROUPED ? a.partial + ((int64_t)blockIdx.x * M + m0) * kPreBN + (n0 - tile_n * kPreBN)
                                : a.partial + (slice * M + m0) * N + n0;
        const int64_t ld = GROUPED ? kPreBN : N;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = i * 32 + j * 8 + lg * 4 + q;
                    if (m0 + r >= M) continue;
                    const uint32_t xs = (uint32_t)__float_as_int(rowinfo[r].x);
                    int32_t* pr = pcol + (int64_t)r * ld;
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        if (col[t]) pr[32 * t] = (int)((uint32_t)acc[i][t][j * 4 + q] - xs);
                }
            }
        }
        return;
    }
    // Non-temporal stores: y is not read again here, so it should not
    // displace the operands from the caches.
    float* ycol = p.y + m0 * N + n0;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = i * 32 + j * 8 + lg * 4 + q;
                if (m0 + r >= M) continue;
                const float2 ri = rowinfo[r];
                const uint32_t xs = (uint32_t)__float_as_int(ri.x);
                float* yr = ycol + (int64_t)r * N;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    if (col[t])
                        __builtin_nontemporal_store(dequant((int)((uint32_t)acc[i][t][j * 4 + q] - xs), ri.y),
                                                    yr + 32 * t);
            }
        }
    }
    if (!p.y_int) return;
    int32_t* yicol = p.y_int + m0 * N + n0;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = i * 32 + j * 8 + lg * 4 + q;
                if (m0 + r >= M) continue;
                const uint32_t xs = (uint32_t)__float_as_int(rowinfo[r].x);
                int32_t* yir = yicol + (int64_t)r * N;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    if (col[t]) __builtin_nontemporal_store((int)((uint32_t)acc[i][t][j * 4 + q] - xs), yir + 32 * t);
            }
        }
    }
}

// Stages of the LDS ring (steps in flight + 1), as measured fastest: three,
// and four for 128 x 256 tiles, whose longer steps give fewer wavefronts per
// SIMD more to hide, and for 32 x 128 tiles, which run on grids too small to
// give each SIMD more than one or two wavefronts (3% over 42 shapes with
// M = 17 .. 128, up to 10% where K or N is long).
constexpr int prefill_stages(int mt, int nt) { return mt == 4 || mt == 1 ? 4 : 3; }

// Column tile of the grouped prefill launch (output rows of W per workgroup).
static int gemm_bn(int64_t M) { (void)M; return kPreBN; }

// Wave tile of a single prefill launch.  Each SIMD runs one wavefront of
// every tile its CU holds, so the time goes as the most tiles any CU gets
// times the MFMA work of one wavefront's tile: ceil(T / CUs) * MT * NT.  Ties
// go to the smaller tile (more resident wavefronts to hide latency), except
// on grids four or more rounds deep, where 128 x 256 tiles (each weight word
// expanded for twice the rows) measure faster.  E.g. on 256 CUs: M = 2048,
// N = 8640 takes 96 x 384 tiles (506 in one round) over 64 x 256 ones (1088:
// up to five per CU); M = 2048, N = 3200 keeps 64 x 256.  Grids that would
// leave CUs idle even with 64 x 256 tiles (batched decode, M = 65 .. a few
// hundred) take 32 x 128 tiles: four times the workgroups, each with a
// quarter of the K loop's MFMAs per step (M = 128, N = 4096, K = 11008:
// 32.7 -> 20.2 us).
struct TileCfg {
    int mt, nt;
};

static TileCfg prefill_tile(int64_t M, int64_t N, int cus) {
    auto rounds = [&](TileCfg t) { return ceil_div(ceil_div(M, 32 * t.mt) * ceil_div(N, 128 * t.nt), cus); };
    const TileCfg small{2, 2}, wide{3, 3}, tall{4, 2}, tiny{1, 1};
    if (ceil_div(M, 64) * ceil_div(N, 256) < cus) return tiny;
    TileCfg best = small;
    int64_t best_cost = rounds(small) * 4;
    if (rounds(wide) * 9 < best_cost) {
        best = wide;
        best_cost = rounds(wide) * 9;
    }
    const int64_t rt = rounds(tall);
    if (rt * 8 < best_cost || (rt * 8 == best_cost && rt >= 4)) best = tall;
    return best;
}

// CUs of the current device, asked of the runtime once per device (the
// query costs more host time than a short prefill launch can hide).
int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

template <int MT, int NT, bool RS>
static void launch_single(GemmArgs& a, hipStream_t stream) {
    a.ntiles_m = ceil_div(a.M, 32 * MT);
    a.ntiles_n = ceil_div(a.p.N, 128 * NT);
    const int64_t S = a.S > 1 ? a.S : 1;
    hipLaunchKernelGGL((gemm_prefill_kernel<MT, NT, false, prefill_stages(MT, NT), RS>),
                       dim3((unsigned)(a.ntiles_m * a.ntiles_n * S)), dim3(256), 0, stream, a);
}

// Split K for grids of 32 x 128 tiles that leave CUs idle over a long K loop
// (batched decode against a wide-K projection, e.g. M = 64, N = 4096,
// K = 11008: 64 tiles for 256 CUs).  Each tile's K loop is cut into S slices
// of whole 128-k steps, one workgroup each; the slices write int32 partial
// sums that the split-K epilogue adds in slice order before dequantizing.
// S comes from a cost estimate fitted to measurements on MI355X: a CU runs
// kStepRate1 128-k steps per us with one resident workgroup (one wavefront
// per SIMD: latency-bound) and kStepRate2 with two or more; a split adds
// kSplitFixedUs (the epilogue launch and the pipeline fill of shorter K
// loops) and 8 bytes per partial element (written, read back) at
// kSplitBytesPerUs.  Candidates keep at most two workgroups per CU and four
// steps per slice.  E.g. M = 96, N = 4096, K = 11008: 96 tiles x 5 slices,
// 22.6 -> 16.3 us; M = 128, N = 8192, K = 28672: 256 tiles x 2 slices,
// 66 -> 45 us; M = 128, N = 8192, K = 8192 stays whole (18 us; 22 us split).
constexpr double kStepRate1 = 3.4;
constexpr double kStepRate2 = 4.4;
constexpr double kSplitFixedUs = 2.0;
constexpr double kSplitBytesPerUs = 4.0e6;
constexpr int64_t kSplitMinSteps = 4;
constexpr int64_t kSplitMaxSlices = 16;

struct SplitCfg {
    int32_t S, sps;   // slices, 128-k steps per slice
};

static double split_cost_us(int64_t M, int64_t N, int64_t tiles, int64_t nsteps, int64_t S, int cus) {
    const int64_t sps = ceil_div(nsteps, S);
    const int64_t per_cu = ceil_div(tiles * ceil_div(nsteps, sps), cus);   // workgroups on the busiest CU
    const double loop = (double)(per_cu * sps) / (per_cu == 1 ? kStepRate1 : kStepRate2);
    return S == 1 ? loop : loop + kSplitFixedUs + 8.0 * (double)S * (double)M * (double)N / kSplitBytesPerUs;
}

static SplitCfg prefill_split(int64_t M, int64_t N, int64_t K, int cus) {
    const TileCfg t = prefill_tile(M, N, cus);
    const int64_t nsteps = ceil_div(ceil_div(K, 64), 2);
    if (t.mt != 1) return {1, (int32_t)nsteps};
    const int64_t tiles = ceil_div(M, 32) * ceil_div(N, 128);
    int64_t best = 1;
    double best_us = split_cost_us(M, N, tiles, nsteps, 1, cus);
    for (int64_t S = 2; S <= kSplitMaxSlices && tiles * S <= 2 * (int64_t)cus && nsteps / S >= kSplitMinSteps; ++S) {
        const double us = split_cost_us(M, N, tiles, nsteps, S, cus);
        if (us < best_us) {
            best = S;
            best_us = us;
        }
    }
    const int64_t sps = ceil_div(nsteps, best);
    return {(int32_t)ceil_div(nsteps, sps), (int32_t)sps};   // no empty slices
}

// Row sums of the int8 activations, xsum[m] = sum_k xq[m][k] in int32
// (wrapping, like the contraction): one wavefront per row, 16 bytes per lane
// per pass (K is a multiple of 16, so no chunk straddles a row end).  Plain
// loads: the contraction reads the same rows next.
__global__ __launch_bounds__(256) void rowsum_kernel(const int8_t* __restrict__ xq, int64_t M, int64_t K,
                                                     int32_t* __restrict__ xsum) {
    const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const int lane = threadIdx.x & 63;
    const int8_t* row = xq + m * K;
    int s = 0;
    for (int64_t k = (int64_t)lane * 16; k < K; k += 1024) {
        const v4i v = *reinterpret_cast<const v4i*>(row + k);
        s = __builtin_amdgcn_sdot4(v.x, 0x01010101, s, false);
        s = __builtin_amdgcn_sdot4(v.y, 0x01010101, s, false);
        s = __builtin_amdgcn_sdot4(v.z, 0x01010101, s, false);
        s = __builtin_amdgcn_sdot4(v.w, 0x01010101, s, false);
    }
    uint32_t u = (uint32_t)s;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) u += (uint32_t)__shfl_xor((int)u, off);
    if (lane == 0) xsum[m] = (int32_t)u;
}

// Either the row sums of the 96 x 384 tile's pre-pass or the split-K
// partials (never both: split K only takes 32 x 128 tiles).
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const SplitCfg sp = prefill_split(M, N, K, device_cus());
    const size_t rows = (size_t)M * sizeof(int32_t);
    const size_t part = sp.S > 1 ? (size_t)sp.S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
    return rows > part ? rows : part;
}

int launch_rowsum(const int8_t* xq, int64_t M, int64_t K, int32_t* xsum, hipStream_t stream) {
    if (M == 0) return BITLINEAR_OK;
    hipLaunchKernelGGL(rowsum_kernel, dim3((unsigned)ceil_div(M, 4)), dim3(256), 0, stream, xq, M, K, xsum);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

// 32 x 128 tiles, split over K when that fills the chip better (the
// partials go to ws, which must not overlap xsum).
template <bool RS>
static int launch_tiny(GemmArgs& a, void* ws, hipStream_t stream) {
    const SplitCfg sp = prefill_split(a.M, a.p.N, a.p.K, device_cus());
    if (sp.S > 1) {
        a.partial = static_cast<int32_t*>(ws);
        a.S = sp.S;
        a.sps = sp.sps;
    }
    launch_single<1, 1, RS>(a, stream);
    BL_LAUNCH_CHECK();
    if (sp.S > 1) return launch_splitk_epilogue(a.partial, sp.S, a.M, a.p, stream);
    return BITLINEAR_OK;
}

int launch_gemm_xsum(const Problem& p, int64_t M, const int32_t* xsum, void* ws, hipStream_t stream) {
    if (!xsum) return BITLINEAR_EINVAL;
    GemmArgs a{};
    a.p = p;
    a.M = M;
    a.xsum = xsum;
    const TileCfg t = prefill_tile(M, p.N, device_cus());
    if (t.mt == 1) return launch_tiny<true>(a, ws, stream);
    if (t.mt == 3) launch_single<3, 3, true>(a, stream);
    else if (t.mt == 4) launch_single<4, 2, true>(a, stream);
    else launch_single<2, 2, true>(a, stream);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

// Without given row sums: the 32 x 128, 64 x 256 and 128 x 256 tiles sum the rows
// from their activation tiles on the way (a few percent of their time);
// the 96 x 384 tile has no registers to spare for that, so a pre-pass sums
// them into the workspace (about M * K bytes read, the operand's first
// pass through the caches).
int launch_gemm(const Problem& p, int64_t M, void* ws, hipStream_t stream) {
    const TileCfg t = prefill_tile(M, p.N, device_cus());
    if (t.mt == 3) {
        int32_t* xsum = static_cast<int32_t*>(ws);
        const int rc = launch_rowsum(p.xq, M, p.K, xsum, stream);
        if (rc) return rc;
        return launch_gemm_xsum(p, M, xsum, nullptr, stream);
    }
    GemmArgs a{};
    a.p = p;
    a.M = M;
    if (t.mt == 1) return launch_tiny<false>(a, ws, stream);
    if (t.mt == 4) launch_single<4, 2, false>(a, stream);
    else launch_single<2, 2, false>(a, stream);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

int gemm_tile_n(int64_t M) { return gemm_bn(M); }

// 17 .. 64 tokens: the streaming MFMA kernel reads each weight once for
// all rows, but its per-step work grows with the token tiles; the 32 x 128
// prefill tiles, split over K where they leave CUs idle, measured faster for
// every shape tried (M = 17 .. 64 against N x K = 4096 x 11008, 11008 x 4096,
// 8192 x 8192, 3200 x 8640, 8192 x 28672, 28672 x 8192; e.g. M = 64,
// N = 4096, K = 11008: 22.5 -> 14.8 us; M = 17, N = 8192, K = 8192 is even).
bool gemm_beats_skinny(int64_t M, int64_t N) {
    (void)N;
    return M > 16;
}

int launch_gemm_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M, bool small,
                        int32_t* partial, hipStream_t stream) {
    // Grouped prefill: 128 x 256 tiles (grid.y = row tiles); plans too small
    // to fill the chip with them take 64 x 256 tiles, some with split K.
    GemmArgs a{};
    a.problems = problems;
    a.units = units;
    a.M = M;
    a.partial = partial;
    if (!small) {
        hipLaunchKernelGGL((gemm_prefill_kernel<4, 2, true, prefill_stages(4, 2), false>),
                           dim3((unsigned)nunits, (unsigned)ceil_div(M, 128)), dim3(256), 0, stream, a);
        BL_LAUNCH_CHECK();
        return BITLINEAR_OK;
    }
    hipLaunchKernelGGL((gemm_prefill_kernel<2, 2, true, prefill_stages(2, 2), false>),
                       dim3((unsigned)nunits, (unsigned)ceil_div(M, 64)), dim3(256), 0, stream, a);
    BL_LAUNCH_CHECK();
    return partial ? launch_grouped_splitk_epilogue(problems, units, nunits, M, kPreBN, partial, stream) : BITLINEAR_OK;
}

}  // namespace bl
