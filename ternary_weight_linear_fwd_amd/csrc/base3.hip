// base3.hip -- decode contraction read straight from the base-3 layout, on the
// gfx950 matrix cores (v_mfma_i32_16x16x64_i8).
//
// The weights: five per byte ([P2] bandwidth paragraph before "Scaling Laws
// and Empirical Benchmarks": 1.58 bits per weight under compact ternary
// packing), 1.6 bits against the 2 bits of the other layout, so a decode pass
// that is bound by weight bytes moves 20% less.  The byte of the layout is
// the fraction form q = ceil(256 v / 243) of the canonical byte
// v = sum_j d_j 3^j (digit d_j = w + 1 of k = 5p + j): q / 256 lies in
// [v / 243, (v + 1) / 243), so for s = 1 .. 5
//     T_s = floor(3^s q / 256) = floor(v / 3^(5 - s))
// is the number formed by the top s digits, and digit 5 - s is
// T_s - 3 T_(s-1) (T_0 = 0).  In a 16-bit lane holding q, multiplying by 3^s
// leaves T_s in the lane's high byte (3^5 * 255 < 2^16): one v_mul_u32_u24
// per digit step and dword gives T_s of two bytes at byte positions 1 and 3.
// With x_s the activation of digit 5 - s,
//     sum_s x_s d_(5-s) = sum_{s=1..5} x_s T_s - 3 sum_{s=1..4} x_(s+1) T_s,
// two linear forms in the T_s: the matrix cores evaluate both at once, with
// token m's activations arranged as A row 2m (x_s against T_s: C0) and row
// 2m + 1 (x_(s+1) against T_s: C1), and zeros against the low bytes of the
// lanes.  T_5 (up to 242) enters as the signed byte T_5 - 128 (the same
// multiply adds 0x8000 to each lane; 128 * sum x_5 is added back).  Then,
// exactly as in the other contraction paths ([P2] "3. Additive Integer
// Accumulation": add on +1, subtract on -1, skip on 0, i.e.
// sum_k x_k (c_k - 1) with c = w + 1),
//     y_int = C0 - 3 C1 + 128 X5 - X,
// X the sum of x over the k-range and X5 that over k = 0 mod 5.  The VALU
// work is 12 operations per 20 weights (two byte splits and ten multiplies),
// against 9 per 16 weights for the 2-bit codes on v_dot4.
//
// Work unit: a workgroup of four wavefronts owns a K-slice of one or more
// consecutive 256-row blocks (a wavefront one 64-row group of the layout per
// block, four 16-column MFMA tiles).  It first arranges the slice's
// activations of up to 8 tokens in LDS (per 80-k block and token, five digit
// steps x 32 bytes plus a zero step); per K-step of four blocks every lane
// then loads its four 16-byte row chunks (row n of each tile, block
// kb + lane / 16: four 256-byte runs per wave load, D steps in flight, the
// stream running on from one row block into the next), splits and
// multiplies them, and issues 40 MFMAs against 10 A fragments read from LDS.
// Lanes whose A row has no token read a zero area.  A finished row block's
// sums go to an LDS stage; the unit writes its outputs at the end as runs of
// consecutive rows.  K-slices leave int32 partial sums for a split-K
// epilogue.
#include "lut.hpp"
#include "xcd.hpp"

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kB3Waves = 4;                    // wavefronts per workgroup
constexpr int kB3Rows = 64 * kB3Waves;         // output rows per workgroup
constexpr int kB3StepLds = 32;                 // one digit step of one block: two 16-byte halves
constexpr int kB3BlockLds = 6 * kB3StepLds;    // five steps and a zero step per block and token
constexpr int kB3BlockX = kBase3BlockK;        // raw activation bytes per block
constexpr int kB3ZeroLds = 256;                // the zero area (A rows without a token)
constexpr int kB3LdsBudget = 48 * 1024;
constexpr int kB3TargetWgs = 768;              // three workgroups per CU (measured best of 384 .. 2048
                                               // on the 70B-shaped projections)
constexpr int kB3Depth = 2;                    // K-steps of weights in flight per wavefront (2 measured
                                               // faster than 3 or 4 at one token)
constexpr int kB3XLoads = 4;                   // 16-byte activation loads per thread: 16 KB per slice

struct B3Args {
    Problem p;          // single problem: p.packed: base-3 layout; p.xq, p.eta: all tokens
    int32_t* partial;   // single problem: [S][M][N] int32 when S > 1
    const Problem* problems;   // grouped: p.Kb = 80-k blocks, p.slices K-slices per 256-row block
    const Unit* units;         // grouped: (problem, 256-row block), K-slices adjacent
    int32_t* gpart;            // grouped, K split: [unit][M][256] int32 partial sums
    int64_t M;          // all tokens
    int32_t m0, mc;     // this pass: tokens m0 .. m0 + mc - 1 (mc <= kBase3MaxTokens)
    int32_t Kb3;        // 80-k blocks along K
    int32_t S, kb_per_slice;
    int32_t row_wgs;    // workgroups along N
    int32_t nblk4;      // LDS blocks per token: kb_per_slice rounded up to whole rings of K-steps
    uint32_t xmagic;    // ceil(2^24 / (nblk4 * 5)): c / (nblk4 * 5) = (c * xmagic) >> 24 for c < 1024
};

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // LDS traffic done (lgkmcnt 0); loads stay in flight
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

// 3^S times both 16-bit lanes of e (bytes q at 0 and 2, zeros at 1 and 3):
// T_S lands in bytes 1 and 3.  For S = 5 each lane also gets 0x8000 added,
// which turns byte 1 and 3 into T_5 - 128 as signed bytes; the carry out of
// the low lane goes into byte 2, the low lane's remainder byte
// (243 q mod 256 <= 242), and stops there.
template <int S>
__device__ __forceinline__ int b3_mul(uint32_t e) {
    if constexpr (S == 1) return (int)__umul24(e, 3u);
    else if constexpr (S == 2) return (int)__umul24(e, 9u);
    else if constexpr (S == 3) return (int)__umul24(e, 27u);
    else if constexpr (S == 4) return (int)__umul24(e, 81u);
    else return (int)(__umul24(e, 243u) + 0x80008000u);
}

// Digit step S of one K-step: two A fragments (halves of the lane's 16-byte
// chunk), one MFMA per tile and half.
template <int S>
__device__ __forceinline__ void b3_digit(const uint32_t (&e)[4][4], const uint32_t (&o)[4][4],
                                         const uint8_t* alds, v4i (&acc)[4]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const v4i A = *reinterpret_cast<const v4i*>(alds + (S - 1) * kB3StepLds + 16 * h);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v4i B;
            B.x = b3_mul<S>(e[t][2 * h]);
            B.y = b3_mul<S>(o[t][2 * h]);
            B.z = b3_mul<S>(e[t][2 * h + 1]);
            B.w = b3_mul<S>(o[t][2 * h + 1]);
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, acc[t], 0, 0, 0);
        }
    }
}

// One K-step: the lane's four row chunks (tile t: row 16t + lane % 16, block
// kb + lane / 16).  Dword d of a chunk holds bytes p = 4d .. 4d + 3; e takes
// bytes 0 and 2 into the low bytes of the two 16-bit lanes, o bytes 1 and 3.
__device__ __forceinline__ void b3_step(const uint4 (&w)[4], const uint8_t* alds, v4i (&acc)[4]) {
    uint32_t e[4][4], o[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t wd[4] = {w[t].x, w[t].y, w[t].z, w[t].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            e[t][d] = wd[d] & 0x00FF00FFu;
            o[t][d] = __builtin_amdgcn_perm(0u, wd[d], 0x0C030C01u);
        }
    }
    b3_digit<1>(e, o, alds, acc);
    b3_digit<2>(e, o, alds, acc);
    b3_digit<3>(e, o, alds, acc);
    b3_digit<4>(e, o, alds, acc);
    b3_digit<5>(e, o, alds, acc);
}

// The lane's chunks of K-step st (blocks past the slice re-read its last
// block: their activations are zero, and the address stays inside the
// layout).
// Non-temporal 16-byte load through a pointer the compiler knows to be
// global: a generic (flat) load counts against both the memory and the LDS
// counters and may return out of order, so the compiler then waits for every
// load in flight before any use.
typedef const __attribute__((address_space(1))) nv_u32x4 b3_gvec;

__device__ __forceinline__ uint4 b3_ldg(const void* p) {
    const nv_u32x4 v = __builtin_nontemporal_load((b3_gvec*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void b3_load(uint4 (&w)[4], const uint8_t* wrow, int64_t b0, int64_t b1, int st,
                                        int lg) {
    int64_t b = b0 + 4 * st + lg;
    if (b >= b1) b = b1 - 1;
    const uint8_t* src = wrow + b * 1024;
#pragma unroll
    for (int t = 0; t < 4; ++t) w[t] = b3_ldg(src + t * 256);
}

template <int D, bool GROUPED>
__global__ __launch_bounds__(256, 2) void base3_mfma_kernel(B3Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lane = t & 63, nl = lane & 15, lg = lane >> 4;
    // Each XCD runs a contiguous run of the workgroups: single problem,
    // neighbouring row blocks of one K-slice, which share its activations in
    // L2; grouped, neighbouring units of the table.
    const uint32_t wg = xcd_contiguous(blockIdx.x, gridDim.x);
    Problem p;
    int64_t rb0, slice, b0, b1, Kb3;
    int nblk4, nrb = 1;   // the unit's 256-row blocks rb0 .. rb0 + nrb - 1
    uint32_t xmagic;
    if constexpr (GROUPED) {
        const Unit un = a.units[wg];
        p = a.problems[un.problem];
        // Split problems: a block's slices are consecutive units from
        // unit_begin on.  Unsplit problems' units may be reordered (the
        // planner runs long K loops first), so their slice is 0 by fiat.
        slice = p.slices > 1 ? (int64_t)wg - p.unit_begin - (int64_t)un.group * p.slices : 0;
        rb0 = (int64_t)un.group * p.blocks_per_unit;
        const int64_t left = ceil_div((int64_t)p.N, kB3Rows) - rb0;
        nrb = left < p.blocks_per_unit ? (int)left : p.blocks_per_unit;
        Kb3 = p.Kb;
        const int64_t kbs = ceil_div(Kb3, p.slices);
        b0 = slice * kbs;
        b1 = b0 + kbs < Kb3 ? b0 + kbs : Kb3;
        nblk4 = (int)ceil_div(kbs, 4 * D) * (4 * D);   // whole rings of K-steps
        xmagic = ((1u << 24) + (uint32_t)(nblk4 * 5) - 1u) / (uint32_t)(nblk4 * 5);
    } else {
        p = a.p;
        rb0 = wg % (uint32_t)a.row_wgs;
        slice = wg / (uint32_t)a.row_wgs;
        Kb3 = a.Kb3;
        b0 = slice * a.kb_per_slice;
        b1 = b0 + a.kb_per_slice < Kb3 ? b0 + a.kb_per_slice : Kb3;
        nblk4 = a.nblk4;
        xmagic = a.xmagic;
    }
    const int64_t N = p.N, K = p.K, G = ceil_div(N, 64);
    const int nblk = (int)(b1 - b0);
    const int nstep_d = ((nblk + 3) / 4 + D - 1) / D * D;   // K-steps per block, padded to whole rings
    const int mc = a.mc;

    // LDS: A arrangement [mc][nblk4][6][2][16], zero area, sums [2][8] (X, X5),
    // raw x [mc][nblk4 * 80], output stage [nrb][mc][256] int32.
    uint8_t* F = lds;
    const uint32_t zero_off = (uint32_t)(mc * nblk4 * kB3BlockLds);
    int* sums = reinterpret_cast<int*>(lds + zero_off + kB3ZeroLds);
    uint32_t* xr = reinterpret_cast<uint32_t*>(lds + zero_off + kB3ZeroLds + 64);
    const int xdw = nblk4 * (kB3BlockX / 4);   // raw dwords per token
    int* ystage = reinterpret_cast<int*>(xr + mc * xdw);

    // The slice's raw activations (up to 16 KB: 4 x 16 bytes per thread) are
    // loaded first, then the first D steps of weights, both as fixed,
    // unconditional load sequences (out-of-range chunks re-read a valid
    // address and are replaced by zeros), so that waiting for the
    // activations leaves the weights in flight.
    const int xch = mc * nblk4 * (kB3BlockX / 16);   // 16-byte activation chunks
    uint4 xv[kB3XLoads];
    bool xin[kB3XLoads];
#pragma unroll
    for (int r = 0; r < kB3XLoads; ++r) {
        const int c = t + 256 * r;
        const int m = (int)(((uint32_t)c * xmagic) >> 24), o = (c - m * (nblk4 * 5)) * 16;
        xin[r] = c < xch && o < nblk * kB3BlockX && b0 * kB3BlockX + o < K;
        xv[r] = b3_ldg(p.xq + (xin[r] ? (int64_t)(a.m0 + m) * K + b0 * kB3BlockX + o : 0));
    }
    // The weight stream runs over the unit's blocks one after the other: step
    // (r, st) is K-step st of block r; past the last step it re-reads that
    // step's chunks (in range, and never used).
    const uint8_t* wbase = reinterpret_cast<const uint8_t*>(p.packed) + nl * 16;
    int lr = 0, ls = 0;   // the next (block, step) to load
    auto load_next = [&](uint4 (&w)[4]) {
        const bool past = lr >= nrb;
        int64_t g = (rb0 + (past ? nrb - 1 : lr)) * kB3Waves + wave;
        if (g >= G) g = G - 1;   // rows past N (a ragged last block): any rows in range
        b3_load(w, wbase + g * Kb3 * 1024, b0, b1, past ? nstep_d - 1 : ls, lg);
        if (!past && ++ls == nstep_d) {
            ls = 0;
            ++lr;
        }
    };
    uint4 wb[D][4];
#pragma unroll
    for (int i = 0; i < D; ++i) load_next(wb[i]);
    if (t < kB3ZeroLds / 4) reinterpret_cast<uint32_t*>(lds + zero_off)[t] = 0u;
    if (t < 16) sums[t] = 0;
#pragma unroll
    for (int r = 0; r < kB3XLoads; ++r)
        if (t + 256 * r < xch) reinterpret_cast<uint4*>(xr)[t + 256 * r] = xin[r] ? xv[r] : make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();

    // X and X5 per token: sums of x over the slice and over its k = 0 mod 5.
    for (int m = 0; m < mc; ++m) {
        int sx = 0, s5 = 0;
        for (int i = t; i < nblk * (kB3BlockX / 4); i += 256) {
            const int v = (int)xr[m * xdw + i];   // 0 past K
            sx = __builtin_amdgcn_sdot4(v, 0x01010101, sx, false);
            // k - 80 b0 = 4i + j is 0 mod 5 for byte j = i mod 5 (when j < 4)
            const int j = i % 5;
            s5 = __builtin_amdgcn_sdot4(v, j < 4 ? 1 << (8 * j) : 0, s5, false);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sx += __shfl_xor(sx, off, 64);
            s5 += __shfl_xor(s5, off, 64);
        }
        if (lane == 0) {
            atomicAdd(&sums[m], sx);
            atomicAdd(&sums[8 + m], s5);
        }
    }

    // A arrangement: dword d of half h of step s (s = 1 .. 5) of block blk
    // pairs with the lane's e/o dword of bytes pa (position 1) and pa + 2
    // (position 3), pa = 8h + {0, 1, 4, 5}[d]; it holds the activations of
    // digit 5 - s of those bytes.  Step 6 is zero (C1 of step 5).
    for (int m = 0; m < mc; ++m) {
        const int8_t* xb = reinterpret_cast<const int8_t*>(xr + m * xdw);
        uint32_t* Fm = reinterpret_cast<uint32_t*>(F) + m * nblk4 * (kB3BlockLds / 4);
        for (int i = t; i < nblk4 * (kB3BlockLds / 4); i += 256) {
            const int blk = i / 48, q = i - blk * 48;
            const int slot = q >> 3, h = (q >> 2) & 1, d = q & 3;
            uint32_t v = 0;
            if (slot < 5) {
                const int s = slot + 1;
                const int pa = 8 * h + ((d & 1) | ((d & 2) << 1));
                const int ka = blk * kB3BlockX + 5 * pa + 5 - s;   // 0 past K
                v = ((uint32_t)(uint8_t)xb[ka] << 8) | ((uint32_t)(uint8_t)xb[ka + 10] << 24);
            }
            Fm[i] = v;
        }
    }
    lds_barrier();

    // Lane (nl, lg): A row nl is token nl / 2, C0 (even) or C1 (odd, one step later).
    const int mt = nl >> 1;
    const bool a_on = mt < mc;
    const uint32_t a_base = a_on ? (uint32_t)((mt * nblk4 + lg) * kB3BlockLds + (nl & 1) * kB3StepLds) : zero_off;
    const uint32_t a_step = a_on ? 4 * kB3BlockLds : 0;

    const bool split = GROUPED ? p.slices > 1 : a.S > 1;
    // This lane's tokens 2 lg + h (h = 0, 1): their sums.
    uint32_t Xh[2], X5h[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int m = 2 * lg + h < mc ? 2 * lg + h : 0;
        Xh[h] = (uint32_t)sums[m];
        X5h[h] = (uint32_t)sums[8 + m];
    }

    v4i acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = v4i{0, 0, 0, 0};
    // A ring of D register stages, refilled unconditionally, so that the loop
    // body is straight-line code and the compiler waits for each stage alone
    // while the later ones stay in flight; the stream runs on from one block
    // into the next (nstep_d, a multiple of D, steps per block: the padding
    // steps meet zero activations).  A finished block's sums go to the LDS
    // output stage, which leaves the loads' count of outstanding operations
    // alone (a global store here would make the next wait drain the stream).
    for (int r = 0; r < nrb; ++r) {
        for (int st0 = 0; st0 < nstep_d; st0 += D) {
#pragma unroll
            for (int i = 0; i < D; ++i) {
                b3_step(wb[i], lds + a_base + (st0 + i) * a_step, acc);
                load_next(wb[i]);
                __builtin_amdgcn_sched_barrier(0);   // the refill leaves here, not at the end of the body
            }
        }
        // Element q of tile t is A row 4 lg + q, column (output row) 16t + nl:
        // token 2 lg + q / 2, C0 for even q, C1 for odd q.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 2 * lg + h;
            if (m >= mc) continue;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                // modulo 2^32: the parts may exceed int32, the result does not
                const int v = (int)((uint32_t)acc[tt][2 * h] - 3u * (uint32_t)acc[tt][2 * h + 1] + 128u * X5h[h] -
                                    Xh[h]);
                ystage[(r * mc + m) * kB3Rows + wave * 64 + tt * 16 + nl] = v;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = v4i{0, 0, 0, 0};
    }
    lds_barrier();

    // The unit's outputs, row runs of consecutive n (rows past N are not
    // stored): dequantized into y (and y_int), or the split partials.
    for (int idx = t; idx < nrb * mc * kB3Rows; idx += 256) {
        const int r = idx / (mc * kB3Rows), rest = idx - r * (mc * kB3Rows);
        const int m = rest / kB3Rows, nloc = rest - m * kB3Rows;
        const int64_t rb = rb0 + r, n = rb * kB3Rows + nloc, mg = a.m0 + m;
        if (n >= N) continue;
        const int v = ystage[idx];
        if (GROUPED && split) {   // split units hold one block
            a.gpart[((int64_t)wg * a.M + mg) * kB3Rows + nloc] = v;
        } else if (split) {
            a.partial[(slice * a.M + mg) * N + n] = v;
        } else {
            p.y[mg * N + n] = dequant(v, dequant_scale(p.eta[mg], p.gamma));
            if (p.y_int) p.y_int[mg * N + n] = v;
        }
    }
}

struct B3Plan {
    int64_t row_wgs;
    int32_t Kb3, S, kb_per_slice, nblk4, mc;
    size_t lds;
};

// Slice lengths are multiples of one ring of K-steps (4 * kB3Depth blocks),
// which is also how far the LDS arrangement of a slice is padded.
constexpr int kB3RingKb = 4 * kB3Depth;

int64_t base3_max_slice_kb(int64_t mc) {
    const int64_t per_blk = mc * (kB3BlockLds + kB3BlockX);
    const int64_t stage = (int64_t)base3_unit_blocks(mc) * mc * kB3Rows * 4;   // the output stage
    int64_t max_kb = (kB3LdsBudget - kB3ZeroLds - 64 - stage) / per_blk / kB3RingKb * kB3RingKb;
    const int64_t max_kb_x = (int64_t)kB3XLoads * 256 * 16 / (mc * kB3BlockX) / kB3RingKb * kB3RingKb;
    if (max_kb > max_kb_x) max_kb = max_kb_x;   // the activation loads cover the slice
    if (max_kb > 2048) max_kb = 2048;   // keeps every MFMA accumulator inside int32
    return max_kb < kB3RingKb ? kB3RingKb : max_kb;
}

static size_t base3_lds_bytes(int64_t mc, int64_t nblk4, int64_t nrb) {
    return (size_t)(mc * nblk4 * (kB3BlockLds + kB3BlockX) + kB3ZeroLds + 64 + nrb * mc * kB3Rows * 4);
}

static B3Plan base3_plan(int64_t M, int64_t N, int64_t K) {
    B3Plan pl;
    pl.Kb3 = (int32_t)ceil_div(K, kBase3BlockK);
    pl.row_wgs = ceil_div(N, kB3Rows);
    pl.mc = (int32_t)(M < kBase3MaxTokens ? (M > 0 ? M : 1) : kBase3MaxTokens);
    const int64_t max_kb = base3_max_slice_kb(pl.mc);
    int64_t S = ceil_div(kB3TargetWgs, pl.row_wgs);
    const int64_t min_s = ceil_div(pl.Kb3, max_kb);
    const int64_t max_s = ceil_div(pl.Kb3, 8);   // at least two K-steps per slice
    if (S > max_s) S = max_s;
    if (S < min_s) S = min_s;
    if (S < 1) S = 1;
    pl.kb_per_slice = (int32_t)ceil_div(pl.Kb3, S);
    pl.S = (int32_t)ceil_div(pl.Kb3, pl.kb_per_slice);
    pl.nblk4 = (int32_t)(ceil_div(pl.kb_per_slice, kB3RingKb) * kB3RingKb);
    pl.lds = base3_lds_bytes(pl.mc, pl.nblk4, 1);
    return pl;
}

size_t base3_ws_bytes(int64_t M, int64_t N, int64_t K) {
    const B3Plan pl = base3_plan(M, N, K);
    return pl.S > 1 ? (size_t)pl.S * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

int launch_base3(const Problem& p, int64_t M, void* ws, hipStream_t stream) {
    if (M == 0) return BITLINEAR_OK;
    const B3Plan pl = base3_plan(M, p.N, p.K);
    B3Args a{};
    a.p = p;
    a.M = M;
    a.Kb3 = pl.Kb3;
    a.S = pl.S;
    a.kb_per_slice = pl.kb_per_slice;
    a.row_wgs = (int32_t)pl.row_wgs;
    a.nblk4 = pl.nblk4;
    a.xmagic = (uint32_t)(((1u << 24) + (uint32_t)(pl.nblk4 * 5) - 1) / (uint32_t)(pl.nblk4 * 5));
    a.partial = pl.S > 1 ? (int32_t*)ws : nullptr;
    const int64_t blocks = pl.row_wgs * pl.S;
    for (int64_t m0 = 0; m0 < M; m0 += kBase3MaxTokens) {
        a.m0 = (int32_t)m0;
        a.mc = (int32_t)(M - m0 < kBase3MaxTokens ? M - m0 : kBase3MaxTokens);
        hipLaunchKernelGGL((base3_mfma_kernel<kB3Depth, false>), dim3((unsigned)blocks), dim3(256), pl.lds, stream, a);
        BL_LAUNCH_CHECK();
    }
    if (pl.S > 1) return launch_splitk_epilogue(a.partial, pl.S, M, p, stream);
    return BITLINEAR_OK;
}

int launch_base3_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                         int64_t max_slice_kb, int32_t* partial, hipStream_t stream) {
    if (M < 1 || M > kBase3MaxTokens) return BITLINEAR_EUNSUPPORTED;
    B3Args a{};
    a.problems = problems;
    a.units = units;
    a.gpart = partial;
    a.M = M;
    a.m0 = 0;
    a.mc = (int32_t)M;
    const size_t lds = base3_lds_bytes(M, ceil_div(max_slice_kb, kB3RingKb) * kB3RingKb, base3_unit_blocks(M));
    hipLaunchKernelGGL((base3_mfma_kernel<kB3Depth, true>), dim3((unsigned)nunits), dim3(256), lds, stream, a);
    BL_LAUNCH_CHECK();
    return partial ? launch_grouped_splitk_epilogue(problems, units, nunits, M, kB3Rows, partial, stream)
                   : BITLINEAR_OK;
}

}  // namespace bl
