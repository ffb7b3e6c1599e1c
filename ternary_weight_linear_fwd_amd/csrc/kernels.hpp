// kernels.hpp -- descriptors and launchers of the gfx950 kernels; the C ABI in
// api.hip validates arguments and calls these.
#pragma once

#include "common.hpp"

namespace bl {

// One row of the grouped quantize stage.
struct QuantRow {
    const float* x;  // [K] float32
    int8_t* xq;      // [K] int8
    float* eta;      // scalar
    int32_t K;
    int32_t pad;
};

// One BitLinear contraction problem as the kernels see it.
struct Problem {
    const int8_t* xq;       // [M][K]
    const float* eta;       // [M]
    const uint4* packed;    // device layout, 16-byte row chunks
    float* y;               // [M][N]
    int32_t* y_int;         // [M][N] or null
    float gamma;
    int32_t N, K;
    int32_t Kb;             // ceil(K / 64)
    int32_t unit_begin;     // first work unit of this problem in a grouped table
    int32_t slices;         // grouped skinny plans: K-slices per 256-row block (1: whole K)
    const float* x;         // [M][K] float32 activations (fused grouped decode), or null
    int32_t blocks_per_unit;  // grouped base-3 plans: 256-row blocks per work unit
    int32_t pad;
};
static_assert(sizeof(Problem) == 80, "Problem descriptor: 80 bytes");

// One work unit of the grouped decode kernel: (problem, 64-row group).
struct Unit {
    int32_t problem;
    int32_t group;
};

// Split-K partial sums of the single-problem decode path.
struct SplitK {
    int32_t* partial;       // [S][M][N] int32, or null when S == 1
    int32_t S;              // number of k-slices
    int32_t kb_per_slice;   // k-blocks per slice
};

// ---- activation quantization (quant.hip)
int launch_quantize(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta, int32_t* xsum,
                    hipStream_t stream);
// nontemporal: x~ stored non-temporally (for contraction kernels that stage
// it through LDS rather than read it through the scalar cache).
int launch_quantize_grouped(const QuantRow* rows, int64_t nrows, bool nontemporal, hipStream_t stream);

// ---- weight quantization and packing (pack.hip)
constexpr int kGammaBins = 256;  // bins[t] collects significands of 2^(t-149) units
size_t gamma_ws_bytes();
int launch_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma_dev,
                        void* ws, hipStream_t stream);
int launch_pack_ternary(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed, int32_t* bad,
                        hipStream_t stream);
int launch_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wt, int32_t* bad,
                  hipStream_t stream);
int launch_fill_zero(void* p, size_t bytes, hipStream_t stream);

// ---- decode contraction, dot4 path for M <= 4 (gemv.hip)
constexpr int kGemvMaxM = 4;
constexpr int kGemvWaves = 4;  // wavefronts (work units) per workgroup
int gemv_split_slices(int64_t M, int64_t N, int64_t K);
size_t gemv_ws_bytes(int64_t M, int64_t N, int64_t K);
int launch_gemv(const Problem& p, int64_t M, void* ws, hipStream_t stream);
// partial: null, or (problems with slices > 1) [unit][M][64] int32 partial
// sums added by launch_grouped_splitk_epilogue (width 64), which follows.
int launch_gemv_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                        int32_t* partial, hipStream_t stream);

// Fused grouped decode for M <= kFusedMaxM tokens on plans too small to fill the chip:
// one workgroup per (problem, 64-row group) quantizes the problem's float32
// rows itself (or copies x~ when the problem has no x), contracts the whole K
// loop across its wavefronts and dequantizes -- one launch, no partial sums
// in memory.  Problems' K at most kFusedMaxK; max_K the longest of them.
constexpr int kFusedMaxK = 16384;
constexpr int kFusedMaxM = 4;
// x~ rows of a fused workgroup in LDS (M * ceil(K / 64) * 64 bytes), at most:
// with the kernel's 8 KB of partial sums a workgroup stays within 64 KB.
constexpr int64_t kFusedMaxLds = 56 * 1024;
int launch_gemv_fused(const Problem* problems, const Unit* units, int64_t nunits, int64_t M, int64_t max_K,
                      hipStream_t stream);
// The same kernel on one problem (row group = workgroup), where
// gemv_fused_single(M, N, K) holds: from x~ (p.x = NULL), or quantizing p.x
// itself (K <= kFusedMaxK; x~ and eta also written to p.xq / p.eta).
bool gemv_fused_single(int64_t M, int64_t N, int64_t K);
int launch_gemv_fused_single(const Problem& p, int64_t M, hipStream_t stream);

// Sum split-K partials [S][M][N] in slice order and apply the dequant epilogue.
int launch_splitk_epilogue(const int32_t* partial, int S, int64_t M, const Problem& p,
                           hipStream_t stream);
// Grouped: problem p's units are its blocks of `width` (64 or 256) output
// rows, each cut into p.slices K-slices (consecutive units); unit u's int32
// sums sit at partial + u * M * width as [m][width].  Adds each block's
// slices in order and dequantizes (problems with p.slices == 1 are left
// alone).
int launch_grouped_splitk_epilogue(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                                   int width, const int32_t* partial, hipStream_t stream);

// ---- decode contraction on int8 MFMA for 4 < M <= 64 (skinny.hip)
constexpr int kSkinnyMaxM = 64;
constexpr int kSkinnyRows = 256;   // output rows per workgroup
int skinny_split_slices(int64_t M, int64_t N, int64_t K);
size_t skinny_ws_bytes(int64_t M, int64_t N, int64_t K);
int launch_skinny(const Problem& p, int64_t M, void* ws, hipStream_t stream);
// Grouped: problem p's units are its 256-row blocks, each cut into
// p.slices K-slices (consecutive units, slice innermost).  With any slices
// > 1, partial holds nunits * M * 256 int32 (unit u's sums at u * M * 256,
// [m][256]) and a second launch adds the slices and dequantizes.
int launch_skinny_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                          int32_t* partial, hipStream_t stream);
constexpr int kSkinnyMaxSlices = 16;   // K-slices per block in a grouped plan, at most
// k-blocks per slice when a block of Kb k-blocks is cut into S slices
// (whole 256-k steps; the planner only picks S that leave no slice empty).
__host__ __device__ inline int64_t skinny_slice_kb(int64_t Kb, int64_t S) {
    return S > 1 ? ((Kb + S - 1) / S + 3) / 4 * 4 : Kb;
}

// ---- prefill contraction on int8 MFMA for M > 64 (gemm.hip; the single
// launch is declared in gemm.hpp)
int gemm_tile_n(int64_t M);  // output rows per workgroup (column tile) for M
// small false: 128 x 256 tiles over whole K loops.  small true: 64 x 256
// tiles; with partial, problem p's K loop in p.slices slices (units and
// partials as for launch_grouped_splitk_epilogue, which follows).
int launch_gemm_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M, bool small,
                        int32_t* partial, hipStream_t stream);

}  // namespace bl
