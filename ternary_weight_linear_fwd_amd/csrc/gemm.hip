// gemm.hip -- ternary x int8 contraction on the gfx950 matrix cores (M > 4).
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
};

template <int MT, int WM, int WN, bool GROUPED>
__global__ __launch_bounds__(64 * WM * WN) void gemm_mfma_kernel(GemmArgs a) {
    constexpr int THREADS = 64 * WM * WN;
    constexpr int BM = WM * 16 * MT;
    constexpr int BN = WN * 64;
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * kLdsRowBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;

    Problem p;
    int64_t tile_n, tile_m;
    if constexpr (GROUPED) {
        const Unit un = a.units[blockIdx.x];
        p = a.problems[un.problem];
        tile_n = un.group;
        tile_m = blockIdx.y;
    } else {
        p = a.p;
        tile_n = blockIdx.x;
        tile_m = blockIdx.y;
    }
    const int64_t M = a.M, N = p.N, K = p.K, Kb = p.Kb;
    const int64_t m0 = tile_m * BM;
    const int64_t Gn = ceil_div(N, 64);
    const int64_t group = tile_n * WN + wn;     // this wave's 64-row group
    const bool group_ok = group < Gn;

    const int nl = lane & 15, lg = lane >> 4;   // MFMA lane coordinates
    v4i acc[MT][4];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][t] = v4i{0, 0, 0, 0};

    const uint4* wbase = p.packed + group * Kb * 64;

    for (int64_t kb = 0; kb < Kb; kb += 4) {
        // ---- B chunks for this step (registers)
        uint4 bch[4];
        const int64_t kbl = kb + lg;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (group_ok && kbl < Kb)
                bch[t] = ldnt_u4(wbase + kbl * 64 + t * 16 + nl);
            else
                bch[t] = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
        }
        // ---- A tile -> LDS
        const int64_t kbase = kb * 64;
        for (int c = tid; c < BM * 16; c += THREADS) {
            const int r = c >> 4, col = c & 15;
            const int64_t m = m0 + r, k = kbase + col * 16;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (m < M && k < K) v = *reinterpret_cast<const uint4*>(p.xq + m * K + k);
            *reinterpret_cast<uint4*>(&lds_a[r * kLdsRowBytes + col * 16]) = v;
        }
        __syncthreads();
        // ---- MFMAs
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            v4i af[MT];
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const int r = wm * 16 * MT + i * 16 + nl;
                af[i] = *reinterpret_cast<const v4i*>(&lds_a[r * kLdsRowBytes + lg * 64 + d * 16]);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t w = d == 0 ? bch[t].x : d == 1 ? bch[t].y : d == 2 ? bch[t].z : bch[t].w;
                v4i bf;
                bf.x = (int)codes_to_ternary(w & 0x03030303u);
                bf.y = (int)codes_to_ternary((w >> 2) & 0x03030303u);
                bf.z = (int)codes_to_ternary((w >> 4) & 0x03030303u);
                bf.w = (int)codes_to_ternary((w >> 6) & 0x03030303u);
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf, acc[i][t], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds rows 4*lg + r (r = 0..3) and column nl of each tile
    if (!group_ok) return;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t m = m0 + wm * 16 * MT + i * 16 + lg * 4 + r;
            if (m >= M) continue;
            const float s = dequant_scale(p.eta[m], p.gamma);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int64_t n = group * 64 + t * 16 + nl;
                if (n >= N) continue;
                const int v = acc[i][t][r];
                p.y[m * N + n] = dequant(v, s);
                if (p.y_int) p.y_int[m * N + n] = v;
            }
        }
    }
}

template <int MT, int WM, int WN>
static int launch_cfg(const GemmArgs& a, int64_t ntn, int64_t ntm, bool grouped, hipStream_t stream) {
    dim3 grid((unsigned)ntn, (unsigned)ntm);
    if (grouped)
        hipLaunchKernelGGL((gemm_mfma_kernel<MT, WM, WN, true>), grid, dim3(64 * WM * WN), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_mfma_kernel<MT, WM, WN, false>), grid, dim3(64 * WM * WN), 0, stream, a);
    BL_LAUNCH_CHECK();
    return BITLINEAR_OK;
}

// Column tile width (output rows of W per workgroup) of the variant used for M.
static int gemm_bn(int64_t M) { return M <= 64 ? 256 : 128; }

static int dispatch(GemmArgs& a, int64_t ntn, bool grouped, hipStream_t stream) {
    const int64_t M = a.M;
    if (M <= 16) return launch_cfg<1, 1, 4>(a, ntn, 1, grouped, stream);
    if (M <= 32) return launch_cfg<2, 1, 4>(a, ntn, 1, grouped, stream);
    if (M <= 64) return launch_cfg<4, 1, 4>(a, ntn, 1, grouped, stream);
    return launch_cfg<4, 2, 2>(a, ntn, ceil_div(M, 128), grouped, stream);
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
