// api.hip -- the C ABI declared in include/bitlinear.h.
//
// Host side only: argument validation (before anything is queued), workspace
// carving, kernel choice by token count and the grouped planner.  All the
// arithmetic of the forward pass runs in the kernels of quant.hip, pack.hip,
// gemv.hip and gemm.hip.  Nothing here allocates device memory.
#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "gemm.hpp"
#include "kernels.hpp"
#include "lut.hpp"
#include "median.hpp"
#include "pack.hpp"
#include "rmsnorm.hpp"

using namespace bl;

// Workspace of the allocation-free fused forward: a fixed device array, one
// copy per GPU that loads the library.  In host code its name is only a
// stand-in, never a device address: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[BITLINEAR_NOALLOC_SCRATCH_BYTES];

namespace bl {
static thread_local char g_last_error[256] = "no error";

void set_hip_error(hipError_t e, const char* where) {
    snprintf(g_last_error, sizeof(g_last_error), "%s (%d) in %s", hipGetErrorName(e), (int)e, where);
}
}  // namespace bl

namespace {

// Clear the process-wide sticky HIP error left by any earlier call outside
// this library before queueing work.
inline void clear_hip_error() { (void)hipGetLastError(); }

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shared size rules: N in [1, 2^31), K in [1, BITLINEAR_MAX_K], K % 16 == 0,
// N*K < 2^40, M in [0, 2^31).
int check_sizes(int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N <= 0 || K <= 0) return BITLINEAR_EINVAL;
    if (M > kMaxDim || N > kMaxDim || K > BITLINEAR_MAX_K) return BITLINEAR_EUNSUPPORTED;
    if (K % 16 != 0) return BITLINEAR_EUNSUPPORTED;
    if (N * K >= (int64_t(1) << 40)) return BITLINEAR_EUNSUPPORTED;
    if (M * K >= (int64_t(1) << 40) || M * N >= (int64_t(1) << 40)) return BITLINEAR_EUNSUPPORTED;
    return BITLINEAR_OK;
}

// Contraction kernel for a single problem: the dot4 GEMV (M <= 4), the
// streaming MFMA decode kernel (M <= 16), or the tiled prefill kernel.
enum class Path { Gemv, Skinny, Tiled };

Path forward_path(int64_t M, int64_t N) {
    if (M <= kGemvMaxM) return Path::Gemv;
    if (M <= kSkinnyMaxM && !gemm_beats_skinny(M, N)) return Path::Skinny;
    return Path::Tiled;
}

size_t forward_ws_bytes(int64_t M, int64_t N, int64_t K) {
    switch (forward_path(M, N)) {
        case Path::Gemv: return gemv_ws_bytes(M, N, K);
        case Path::Skinny: return skinny_ws_bytes(M, N, K);
        default: return gemm_ws_bytes(M, N, K);
    }
}

Problem make_problem(const int8_t* xq, const float* eta, const uint8_t* packed, float gamma,
                     int64_t N, int64_t K, float* y, int32_t* y_int, const float* x = nullptr) {
    Problem p{};
    p.x = x;
    p.xq = xq;
    p.eta = eta;
    p.packed = reinterpret_cast<const uint4*>(packed);
    p.y = y;
    p.y_int = y_int;
    p.gamma = gamma;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.Kb = (int32_t)ceil_div(K, 64);
    p.slices = 1;
    return p;
}

// xsum (may be null): the activation row sums for the prefill kernel, which
// otherwise sums them itself (or into the workspace first).  The decode
// kernels sum their slices themselves.
int run_forward(const int8_t* xq, const float* eta, const int32_t* xsum, const uint8_t* packed,
                float gamma, int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int, void* ws,
                hipStream_t stream) {
    if (M == 0) return BITLINEAR_OK;
    const Problem p = make_problem(xq, eta, packed, gamma, N, K, y, y_int);
    switch (forward_path(M, N)) {
        case Path::Gemv: return launch_gemv(p, M, ws, stream);
        case Path::Skinny: return launch_skinny(p, M, ws, stream);
        default: return xsum ? launch_gemm_xsum(p, M, xsum, ws, stream) : launch_gemm(p, M, ws, stream);
    }
}

// Workspace of the fused float32 forward: xq, eta, the row sums (prefill
// kernel only; the quantizer fills them), then the contraction's own
// workspace.
struct F32Ws {
    size_t xq, eta, xsum, bytes;
};

F32Ws f32_ws(int64_t M, int64_t N, int64_t K) {
    F32Ws w;
    w.xq = align256((size_t)(M * K));
    w.eta = align256((size_t)(4 * M));
    w.xsum = forward_path(M, N) == Path::Tiled ? align256((size_t)(4 * M)) : 0;
    w.bytes = w.xq + w.eta + w.xsum + align256(forward_ws_bytes(M, N, K));
    return w;
}

// Contraction kernel of a grouped plan: 0 dot4 GEMV, 1 prefill MFMA (128 x
// 256 tiles), 2 skinny MFMA, 3 skinny MFMA with K split, 4 prefill MFMA
// (64 x 256 tiles) with K split (split plans: partials in the table, then an
// epilogue), 5 prefill MFMA (64 x 256 tiles), 6 dot4 GEMV with K split,
// 7 fused dot4 GEMV (quantize + contract + dequant in one launch, whole K
// per workgroup; no quantize stage), 8 base-3 matrix-core decode over
// 256-row blocks, 9 the same with K split.
constexpr int32_t kPlanGemv = 0, kPlanGemm = 1, kPlanSkinny = 2, kPlanSkinnySplit = 3, kPlanGemmSplit = 4,
                  kPlanGemmSmall = 5, kPlanGemvSplit = 6, kPlanGemvFused = 7, kPlanBase3 = 8,
                  kPlanBase3Split = 9, kPlanLast = 9;

struct TableLayout {
    size_t problems_off, units_off, rows_off, part_off, bytes;
};

// The work table: problem descriptors, work units, quantizer rows and, for
// split plans, the partial sums (M x 256 int32 per unit).
TableLayout table_layout(int64_t count, int64_t nunits, int64_t nrows, int32_t kernel, int64_t M) {
    TableLayout t;
    t.problems_off = 0;
    t.units_off = align256((size_t)count * sizeof(Problem));
    t.rows_off = t.units_off + align256((size_t)nunits * sizeof(Unit));
    t.part_off = t.rows_off + align256((size_t)nrows * sizeof(QuantRow));
    const size_t width = kernel == kPlanGemvSplit ? 64   // output rows per work unit
                         : (kernel == kPlanSkinnySplit || kernel == kPlanGemmSplit || kernel == kPlanBase3Split)
                             ? kSkinnyRows
                             : 0;
    const size_t part = (size_t)nunits * (size_t)M * width * sizeof(int32_t);
    t.bytes = t.part_off + align256(part);
    return t;
}

// Work units of the grouped contraction for one problem (before K slices).
int64_t problem_units(int32_t kernel, int64_t M, int64_t N) {
    if (kernel == kPlanGemv || kernel == kPlanGemvFused) return ceil_div(N, 64);   // per 64-row group
    if (kernel == kPlanGemm) return ceil_div(N, gemm_tile_n(M));
    return ceil_div(N, kSkinnyRows);                   // one workgroup per 256 rows (skinny, base-3)
}

int32_t plan_kernel(int64_t M) {
    if (M <= kGemvMaxM) return kPlanGemv;
    if (M <= kSkinnyMaxM) return kPlanSkinny;
    return kPlanGemm;
}

// K-slices per 256-row block for a grouped skinny plan.  Plans whose blocks
// alone leave CUs idle (a single transformer block at a few dozen tokens:
// 166 blocks for hidden 4096 / FFN 11008) cut every problem's K loop into
// slices of about the same length, aiming at two workgroups per CU up to 32
// tokens and one above (the partials grow with M), with at least
// kGroupedSplitMinSteps 256-k steps per slice; the slices write int32
// partials that a second launch adds in slice order.  Large plans (a whole
// model's projections) keep whole K loops.  Measured on the seven
// projections of a hidden-4096 / FFN-11008 block: M = 8 43 -> 20 us,
// M = 32 50 -> 31 us, M = 64 68 -> 49 us.
constexpr int64_t kGroupedSplitMinSteps = 2;
constexpr int64_t kGroupedSplitMaxSlices = kSkinnyMaxSlices;

void choose_slices(std::vector<Problem>& problems, int64_t M, int cus) {
    const int64_t wg_per_cu = M <= 32 ? 2 : 1;
    int64_t blocks = 0, work = 0;   // work: 256-row blocks x 256-k steps
    for (const Problem& p : problems) {
        blocks += ceil_div(p.N, kSkinnyRows);
        work += ceil_div(p.N, kSkinnyRows) * ceil_div(p.Kb, 4);
    }
    if (blocks >= cus) return;
    int64_t len = ceil_div(work, wg_per_cu * cus);   // steps per slice
    if (len < kGroupedSplitMinSteps) len = kGroupedSplitMinSteps;
    for (Problem& p : problems) {
        int64_t S = ceil_div(ceil_div(p.Kb, 4), len);
        if (S > kGroupedSplitMaxSlices) S = kGroupedSplitMaxSlices;
        while (S > 1 && (S - 1) * skinny_slice_kb(p.Kb, S) >= p.Kb) --S;   // no empty slice
        p.slices = (int32_t)(S < 1 ? 1 : S);
    }
}

// A grouped prefill plan past 64 tokens whose 128 x 256 tiles would not give
// every CU kGemmSmallBelow of them (one block at 65 .. a few hundred tokens)
// takes 64 x 256 tiles instead, and problems with long K loops are cut into
// slices of about equal length (whole 128-k steps, at least
// kGemmSplitMinSteps), aiming at three workgroups per two CUs.  Few slices
// measured best (the partials cost more than a deeper grid gains), so only
// the long projections split: hidden 4096 / FFN 11008 at M = 128, the down
// projection in three.  Returns whether the plan is small; slices > 1
// where a problem is split.
constexpr int64_t kGemmSmallBelow = 2;
constexpr int64_t kGemmSplitMinSteps = 32;

bool choose_gemm_slices(std::vector<Problem>& problems, int64_t M, int cus) {
    int64_t big = 0, work = 0;   // work: 64 x 256 tiles x 128-k steps
    for (const Problem& p : problems) {
        big += ceil_div(p.N, 256) * ceil_div(M, 128);
        work += ceil_div(p.N, 256) * ceil_div(M, 64) * ceil_div(p.Kb, 2);
    }
    if (big >= kGemmSmallBelow * cus) return false;
    int64_t len = ceil_div(2 * work, 3 * (int64_t)cus);   // steps per slice
    if (len < kGemmSplitMinSteps) len = kGemmSplitMinSteps;
    for (Problem& p : problems) {
        const int64_t nsteps = ceil_div(p.Kb, 2);
        int64_t S = ceil_div(nsteps, len);
        if (S > kGroupedSplitMaxSlices) S = kGroupedSplitMaxSlices;
        while (S > 1 && (S - 1) * ceil_div(nsteps, S) >= nsteps) --S;   // no empty slice
        p.slices = (int32_t)(S < 1 ? 1 : S);
    }
    return true;
}

constexpr int64_t kSmallPlanTiledFromM = 17;

// K-slices per 64-row group for a grouped dot4 plan (M <= 4) whose groups
// alone give the chip fewer than kGemvSmallWaves wavefronts (one transformer
// block: 520 groups for hidden 3200 / FFN 8640), cut into slices of about
// equal length aiming at kGemvSplitWaves wavefronts, at least
// kGemvSplitMinKb k-blocks each.
constexpr int64_t kGemvSmallWaves = 8192;
constexpr int64_t kGemvSplitWaves = 4096;
constexpr int64_t kGemvSplitMinKb = 8;

// A dot4 plan of at most kFusedMaxM tokens whose 64-row groups give the chip
// fewer than kGemvSmallWaves wavefronts, and whose K fits the fused kernel's
// LDS, takes the fused kernel: one workgroup per group quantizes, contracts
// the whole K loop and dequantizes.
bool fused_gemv_plan(const std::vector<Problem>& problems, int64_t M) {
    if (M <= 0 || M > kFusedMaxM) return false;
    int64_t groups = 0;
    for (const Problem& p : problems) {
        if (p.K > kFusedMaxK || M * ceil_div(p.K, 64) * 64 > kFusedMaxLds) return false;
        groups += ceil_div(p.N, 64);
    }
    return groups < kGemvSmallWaves;
}

bool choose_gemv_slices(std::vector<Problem>& problems) {
    int64_t groups = 0, work = 0;   // work: 64-row groups x k-blocks
    for (const Problem& p : problems) {
        groups += ceil_div(p.N, 64);
        work += ceil_div(p.N, 64) * p.Kb;
    }
    if (groups >= kGemvSmallWaves) return false;
    int64_t len = ceil_div(work, kGemvSplitWaves);
    if (len < kGemvSplitMinKb) len = kGemvSplitMinKb;
    bool any = false;
    for (Problem& p : problems) {
        int64_t S = ceil_div(p.Kb, len);
        if (S > kSkinnyMaxSlices) S = kSkinnyMaxSlices;
        while (S > 1 && (S - 1) * ceil_div(p.Kb, S) >= p.Kb) --S;   // no empty slice
        p.slices = (int32_t)(S < 1 ? 1 : S);
        any = any || p.slices > 1;
    }
    return any;
}

// K-slices for a grouped base-3 plan.  Every slice fits the kernel's LDS
// arrangement (base3_max_slice_kb); plans whose 256-row blocks number fewer
// than kBase3GroupedUnits (one transformer block, say) are cut further into
// slices of about equal length aiming at that many work units, at least
// kBase3SplitMinKb blocks of 80 k each.
constexpr int64_t kBase3GroupedUnits = 768;
constexpr int64_t kBase3SplitMinKb = 8;
// Problems whose K loop is not split run base3_unit_blocks(M) consecutive
// 256-row blocks per work unit: one arrangement of the activations in LDS and
// one unbroken weight stream serve them all (split problems: one block per
// unit, the layout of the split partials).

bool choose_base3_slices(std::vector<Problem>& problems, int64_t M) {
    const int64_t mc = M < 1 ? 1 : (M > kBase3MaxTokens ? kBase3MaxTokens : M);
    const int64_t max_kb = base3_max_slice_kb(mc);
    int64_t blocks = 0, work = 0;   // work: 256-row blocks x 80-k blocks
    for (const Problem& p : problems) {
        blocks += ceil_div(p.N, kSkinnyRows);
        work += ceil_div(p.N, kSkinnyRows) * p.Kb;
    }
    int64_t len = max_kb;
    if (blocks < kBase3GroupedUnits) {
        len = ceil_div(work, kBase3GroupedUnits);
        if (len < kBase3SplitMinKb) len = kBase3SplitMinKb;
        if (len > max_kb) len = max_kb;
    }
    bool any = false;
    for (Problem& p : problems) {
        int64_t S = ceil_div(p.Kb, len);
        while (S > 1 && (S - 1) * ceil_div(p.Kb, S) >= p.Kb) --S;   // no empty slice
        p.slices = (int32_t)(S < 1 ? 1 : S);
        p.blocks_per_unit = p.slices > 1 ? 1 : base3_unit_blocks(mc);
        any = any || p.slices > 1;
    }
    return any;
}

struct PlanHost {
    std::vector<Problem> problems;
    std::vector<Unit> units;
    std::vector<QuantRow> rows;
    int32_t kernel = kPlanGemv;
};

// Work-unit order of unsplit plans.  A grouped grid holds far more
// workgroups than the chip runs at once, and each XCD works through its
// contiguous run of the grid (xcd_contiguous) in order; units whose K loops
// start late decide when the launch ends.  Within each XCD's run the units
// therefore go longest first (stable: a problem's units stay adjacent), so
// the run ends on short units.  Plans whose kernel takes units[blockIdx.x]
// (round-robin over the XCDs) are ordered as one run.  Measured on the
// 70B-shaped decode sweep: 2% at one token, 3% at 16 tokens.  Split plans
// keep their order: a block's K-slices are found from the unit index.
void order_longest_first(PlanHost& h, int64_t units_per_wg, bool xcd_runs) {
    const int64_t n = (int64_t)h.units.size();
    auto length = [&h](const Unit& u) {
        const Problem& p = h.problems[u.problem];
        int64_t rows = 1;   // 256-row blocks of a base-3 unit
        if (p.blocks_per_unit > 1) {
            const int64_t left = ceil_div(p.N, kSkinnyRows) - (int64_t)u.group * p.blocks_per_unit;
            rows = left < p.blocks_per_unit ? left : p.blocks_per_unit;
        }
        return (int64_t)p.Kb * rows;
    };
    auto longer = [&length](const Unit& a, const Unit& b) { return length(a) > length(b); };
    if (!xcd_runs) {
        std::stable_sort(h.units.begin(), h.units.end(), longer);
        return;
    }
    // The XCD runs as xcd_contiguous cuts a grid of T workgroups.
    constexpr int64_t X = 8;
    const int64_t T = ceil_div(n, units_per_wg), q = T / X, r = T % X;
    for (int64_t x = 0; x < X; ++x) {
        const int64_t b0 = x * q + (x < r ? x : r), b1 = b0 + q + (x < r ? 1 : 0);
        const int64_t u0 = b0 * units_per_wg, u1 = b1 * units_per_wg < n ? b1 * units_per_wg : n;
        if (u0 < u1) std::stable_sort(h.units.begin() + u0, h.units.begin() + u1, longer);
    }
}

int build_plan(const bitlinear_problem* pr, int32_t count, int64_t M, PlanHost& out) {
    if (!pr || count <= 0 || M < 0 || M > kMaxDim) return BITLINEAR_EINVAL;
    std::map<const int8_t*, const float*> xq_source;  // xq buffer -> its x
    for (int32_t i = 0; i < count; ++i) {
        const bitlinear_problem& q = pr[i];
        if (q.format != kFormat2Bit && q.format != kFormatBase3) return BITLINEAR_EINVAL;
        if (q.format != pr[0].format) return BITLINEAR_EINVAL;   // one layout per plan
        int rc = check_sizes(M, q.N, q.K);
        if (rc) return rc;
        if (!q.packed || !q.y || !q.xq || !q.eta) return BITLINEAR_EINVAL;
        if (!aligned(q.packed, 16) || !aligned(q.xq, 16) || (q.x && !aligned(q.x, 16)))
            return BITLINEAR_EINVAL;
        auto it = xq_source.find(q.xq);
        if (it == xq_source.end()) {
            xq_source[q.xq] = q.x;
            if (q.x) {
                for (int64_t m = 0; m < M; ++m) {
                    QuantRow r{};
                    r.x = q.x + m * q.K;
                    r.xq = q.xq + m * q.K;
                    r.eta = q.eta + m;
                    r.K = q.K;
                    out.rows.push_back(r);
                }
            }
        } else if (it->second != q.x) {
            return BITLINEAR_EINVAL;  // one xq buffer fed from two different sources
        }
        out.problems.push_back(make_problem(q.xq, q.eta, q.packed, q.gamma, q.N, q.K, q.y, q.y_int, q.x));
    }
    if (pr[0].format == kFormatBase3) {
        if (M > kBase3MaxTokens) return BITLINEAR_EUNSUPPORTED;
        for (Problem& p : out.problems) p.Kb = (int32_t)ceil_div(p.K, kBase3BlockK);
        out.kernel = choose_base3_slices(out.problems, M) ? kPlanBase3Split : kPlanBase3;
    } else {
        out.kernel = plan_kernel(M);
    }
    if (out.kernel == kPlanGemv && fused_gemv_plan(out.problems, M)) {
        out.kernel = kPlanGemvFused;
        out.rows.clear();   // each workgroup quantizes its problem's rows itself
    }
    if (out.kernel == kPlanGemv && M > 0 && choose_gemv_slices(out.problems)) out.kernel = kPlanGemvSplit;
    if (out.kernel == kPlanSkinny && M >= kSmallPlanTiledFromM) {
        // Small plans take the 64 x 256 prefill tiles from kSmallPlanTiledFromM
        // tokens on (every 64-row tile then at least half used).
        std::vector<Problem> trial = out.problems;
        if (choose_gemm_slices(trial, M, device_cus())) {
            out.problems = trial;
            out.kernel = kPlanGemmSmall;
            for (const Problem& p : out.problems)
                if (p.slices > 1) out.kernel = kPlanGemmSplit;
        }
    }
    if (out.kernel == kPlanSkinny && M > 0) {
        choose_slices(out.problems, M, device_cus());
        for (const Problem& p : out.problems)
            if (p.slices > 1) out.kernel = kPlanSkinnySplit;
    }
    if (out.kernel == kPlanGemm && choose_gemm_slices(out.problems, M, device_cus())) {
        out.kernel = kPlanGemmSmall;
        for (const Problem& p : out.problems)
            if (p.slices > 1) out.kernel = kPlanGemmSplit;
    }
    // Units: each problem's blocks in order, the K-slices of a block adjacent.
    for (int32_t i = 0; i < count; ++i) {
        Problem& p = out.problems[i];
        p.unit_begin = (int32_t)out.units.size();
        const int32_t k = out.kernel == kPlanSkinnySplit ? kPlanSkinny
                          : (out.kernel == kPlanGemmSplit || out.kernel == kPlanGemmSmall) ? kPlanGemm
                          : out.kernel == kPlanGemvSplit                                  ? kPlanGemv
                          : out.kernel == kPlanBase3Split                                 ? kPlanBase3
                                                                                          : out.kernel;
        const int64_t nu = k == kPlanBase3 ? ceil_div(ceil_div(p.N, kSkinnyRows), p.blocks_per_unit)
                                           : problem_units(k, M, p.N);
        for (int64_t g = 0; g < nu; ++g)
            for (int32_t s = 0; s < p.slices; ++s) out.units.push_back(Unit{i, (int32_t)g});
        if (out.units.size() >= (size_t)kMaxDim) return BITLINEAR_EUNSUPPORTED;
    }
    if (out.kernel == kPlanGemv) order_longest_first(out, kGemvWaves, true);
    if (out.kernel == kPlanSkinny || out.kernel == kPlanBase3) order_longest_first(out, 1, true);
    if (out.kernel == kPlanGemvFused) order_longest_first(out, 1, false);
    // Quantizer rows, one workgroup each in grid order: longest first too.
    std::stable_sort(out.rows.begin(), out.rows.end(), [](const QuantRow& a, const QuantRow& b) { return a.K > b.K; });
    return BITLINEAR_OK;
}

// Device addresses of `scratch` (top of this file), one per device, looked up on a
// device's first allocation-free call.
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mutex;

// The device address of `scratch` on the current device, or null after a
// failed lookup (the HIP error is recorded for bitlinear_last_error()).
void* scratch_for_current_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kScratchDevices) {
        bl::set_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice, "hipGetDevice (scratch lookup)");
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
        bl::set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

const char* bitlinear_status_string(int status) {
    switch (status) {
        case BITLINEAR_OK: return "BITLINEAR_OK";
        case BITLINEAR_EINVAL: return "BITLINEAR_EINVAL: invalid argument";
        case BITLINEAR_EUNSUPPORTED: return "BITLINEAR_EUNSUPPORTED: unsupported size";
        case BITLINEAR_EWORKSPACE: return "BITLINEAR_EWORKSPACE: workspace too small";
        case BITLINEAR_EBADCODE: return "BITLINEAR_EBADCODE: value outside {-1, 0, 1}";
        case BITLINEAR_EHIP: return "BITLINEAR_EHIP: HIP runtime error";
        default: return "BITLINEAR_UNKNOWN";
    }
}

int bitlinear_abi_version(void) { return 10200; }

const char* bitlinear_last_error(void) { return g_last_error; }

size_t bitlinear_packed_bytes(int64_t N, int64_t K) {
    if (check_sizes(0, N, K) != BITLINEAR_OK) return 0;
    return (size_t)(ceil_div(N, 64) * ceil_div(K, 64) * kBlockBytes);
}

size_t bitlinear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_sizes(M, N, K) != BITLINEAR_OK) return 0;
    const size_t f32 = f32_ws(M, N, K).bytes;
    size_t pack = align256(gamma_ws_bytes());
    if (align256(median_ws_bytes()) > pack) pack = align256(median_ws_bytes());
    return f32 > pack ? f32 : pack;
}

int bitlinear_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                           int32_t* xsum, void* stream) {
    int rc = check_sizes(M, 1, K);
    if (rc) return rc;
    if (!x || !xq || !eta) return BITLINEAR_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 16)) return BITLINEAR_EINVAL;
    clear_hip_error();
    return launch_quantize(x, M, K, xq, eta, xsum, (hipStream_t)stream);
}

int bitlinear_rmsnorm_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                                   int32_t* xsum, float* ms, void* stream) {
    int rc = check_sizes(M, 1, K);
    if (rc) return rc;
    if (!x || !xq || !eta) return BITLINEAR_EINVAL;
    if (!aligned(x, 16) || !aligned(xq, 16)) return BITLINEAR_EINVAL;
    clear_hip_error();
    return launch_rmsnorm_quantize(x, M, K, xq, eta, xsum, ms, (hipStream_t)stream);
}

int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                           float* gamma_host, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!W || !packed) return BITLINEAR_EINVAL;
    if (!aligned(W, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    if (!ws || !aligned(ws, 256) || ws_bytes < gamma_ws_bytes()) return BITLINEAR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    clear_hip_error();
    rc = launch_pack_weights(W, N, K, packed, gamma, ws, s);
    if (rc) return rc;
    if (gamma_host) {
        const float* g = (const float*)((const char*)ws + kGammaBins * sizeof(unsigned long long));
        BL_HIP_CHECK(hipMemcpyAsync(gamma_host, g, sizeof(float), hipMemcpyDeviceToHost, s));
        BL_HIP_CHECK(hipStreamSynchronize(s));
    }
    return BITLINEAR_OK;
}

int bitlinear_pack_weights_absmedian(const float* W, int64_t N, int64_t K, uint8_t* packed,
                                     float* gamma, float* gamma_host, void* ws, size_t ws_bytes,
                                     void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!W || !packed) return BITLINEAR_EINVAL;
    if (!aligned(W, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    if (!ws || !aligned(ws, 256) || ws_bytes < median_ws_bytes()) return BITLINEAR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    clear_hip_error();
    const float* g = nullptr;
    rc = launch_pack_weights_absmedian(W, N, K, packed, gamma, ws, &g, s);
    if (rc) return rc;
    if (gamma_host) {
        BL_HIP_CHECK(hipMemcpyAsync(gamma_host, g, sizeof(float), hipMemcpyDeviceToHost, s));
        BL_HIP_CHECK(hipStreamSynchronize(s));
    }
    return BITLINEAR_OK;
}

int bitlinear_pack_ternary(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed, int32_t* bad,
                           void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!Wt || !packed) return BITLINEAR_EINVAL;
    if (!aligned(Wt, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    clear_hip_error();
    if (bad && (rc = launch_zero_i32(bad, (hipStream_t)stream))) return rc;
    return launch_pack_ternary(Wt, N, K, packed, bad, (hipStream_t)stream);
}

int bitlinear_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wt, int32_t* bad,
                             void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!Wt || !packed) return BITLINEAR_EINVAL;
    if (!aligned(Wt, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    clear_hip_error();
    if (bad && (rc = launch_zero_i32(bad, (hipStream_t)stream))) return rc;
    return launch_unpack(packed, N, K, Wt, bad, (hipStream_t)stream);
}

size_t bitlinear_packed3_bytes(int64_t N, int64_t K) {
    if (check_sizes(0, N, K) != BITLINEAR_OK) return 0;
    return packed3_bytes(N, K);
}

int bitlinear_pack_weights3(const float* W, int64_t N, int64_t K, uint8_t* packed3, float* gamma,
                            float* gamma_host, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!W || !packed3) return BITLINEAR_EINVAL;
    if (!aligned(W, 16) || !aligned(packed3, 16)) return BITLINEAR_EINVAL;
    if (!ws || !aligned(ws, 256) || ws_bytes < gamma_ws_bytes()) return BITLINEAR_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    clear_hip_error();
    rc = launch_pack_weights3(W, N, K, packed3, gamma, ws, s);
    if (rc) return rc;
    if (gamma_host) {
        const float* g = (const float*)((const char*)ws + kGammaBins * sizeof(unsigned long long));
        BL_HIP_CHECK(hipMemcpyAsync(gamma_host, g, sizeof(float), hipMemcpyDeviceToHost, s));
        BL_HIP_CHECK(hipStreamSynchronize(s));
    }
    return BITLINEAR_OK;
}

int bitlinear_pack_ternary3(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed3, int32_t* bad,
                            void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!Wt || !packed3) return BITLINEAR_EINVAL;
    if (!aligned(packed3, 16)) return BITLINEAR_EINVAL;
    clear_hip_error();
    if (bad && (rc = launch_zero_i32(bad, (hipStream_t)stream))) return rc;
    return launch_pack_ternary3(Wt, N, K, packed3, bad, (hipStream_t)stream);
}

int bitlinear_unpack_weights3(const uint8_t* packed3, int64_t N, int64_t K, int8_t* Wt,
                              int32_t* bad, void* stream) {
    int rc = check_sizes(0, N, K);
    if (rc) return rc;
    if (!Wt || !packed3) return BITLINEAR_EINVAL;
    if (!aligned(packed3, 16)) return BITLINEAR_EINVAL;
    clear_hip_error();
    if (bad && (rc = launch_zero_i32(bad, (hipStream_t)stream))) return rc;
    return launch_unpack3(packed3, N, K, Wt, bad, (hipStream_t)stream);
}

size_t bitlinear_lut_workspace_bytes(int64_t M, int64_t N, int64_t K, int format) {
    if (check_sizes(M, N, K) != BITLINEAR_OK) return 0;
    if (format != kFormat2Bit && format != kFormatBase3) return 0;
    return align256(lut_ws_bytes(M, N, K, format));
}

int bitlinear_forward_lut(const int8_t* xq, const float* eta, const uint8_t* packed, int format,
                          float gamma, int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int,
                          void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(M, N, K);
    if (rc) return rc;
    if (format != kFormat2Bit && format != kFormatBase3) return BITLINEAR_EINVAL;
    if (!xq || !eta || !packed || !y) return BITLINEAR_EINVAL;
    if (!aligned(packed, 16)) return BITLINEAR_EINVAL;
    const size_t need = lut_ws_bytes(M, N, K, format);
    if (need && (!ws || !aligned(ws, 256) || ws_bytes < need)) return BITLINEAR_EWORKSPACE;
    if (M == 0) return BITLINEAR_OK;
    clear_hip_error();
    Problem p = make_problem(xq, eta, packed, gamma, N, K, y, y_int);
    return launch_lut(p, M, format, ws, (hipStream_t)stream);
}

size_t bitlinear_forward3_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_sizes(M, N, K) != BITLINEAR_OK) return 0;
    return align256(base3_ws_bytes(M, N, K));
}

int bitlinear_forward3(const int8_t* xq, const float* eta, const uint8_t* packed3, float gamma,
                       int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int, void* ws,
                       size_t ws_bytes, void* stream) {
    int rc = check_sizes(M, N, K);
    if (rc) return rc;
    if (!xq || !eta || !packed3 || !y) return BITLINEAR_EINVAL;
    if (!aligned(xq, 16) || !aligned(packed3, 16)) return BITLINEAR_EINVAL;
    const size_t need = base3_ws_bytes(M, N, K);
    if (need && (!ws || !aligned(ws, 256) || ws_bytes < need)) return BITLINEAR_EWORKSPACE;
    if (M == 0) return BITLINEAR_OK;
    clear_hip_error();
    Problem p = make_problem(xq, eta, packed3, gamma, N, K, y, y_int);
    return launch_base3(p, M, ws, (hipStream_t)stream);
}

int bitlinear_forward(const int8_t* xq, const float* eta, const uint8_t* packed, float gamma,
                      int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int, void* ws,
                      size_t ws_bytes, void* stream) {
    int rc = check_sizes(M, N, K);
    if (rc) return rc;
    if (!xq || !eta || !packed || !y) return BITLINEAR_EINVAL;
    if (!aligned(xq, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    const size_t need = forward_ws_bytes(M, N, K);
    if (need && (!ws || !aligned(ws, 256) || ws_bytes < need)) return BITLINEAR_EWORKSPACE;
    clear_hip_error();
    return run_forward(xq, eta, nullptr, packed, gamma, M, N, K, y, y_int, ws, (hipStream_t)stream);
}

int bitlinear_forward_xsum(const int8_t* xq, const float* eta, const int32_t* xsum,
                           const uint8_t* packed, float gamma, int64_t M, int64_t N, int64_t K,
                           float* y, int32_t* y_int, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_sizes(M, N, K);
    if (rc) return rc;
    if (!xq || !eta || !xsum || !packed || !y) return BITLINEAR_EINVAL;
    if (!aligned(xq, 16) || !aligned(packed, 16) || !aligned(xsum, 4)) return BITLINEAR_EINVAL;
    const size_t need = forward_ws_bytes(M, N, K);
    if (need && (!ws || !aligned(ws, 256) || ws_bytes < need)) return BITLINEAR_EWORKSPACE;
    clear_hip_error();
    return run_forward(xq, eta, xsum, packed, gamma, M, N, K, y, y_int, ws, (hipStream_t)stream);
}

static int forward_f32_common(const float* x, const uint8_t* packed, float gamma, int64_t M,
                              int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                              void* stream, bool rmsnorm) {
    int rc = check_sizes(M, N, K);
    if (rc) return rc;
    if (!x || !packed || !y) return BITLINEAR_EINVAL;
    if (!aligned(x, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    const F32Ws w = f32_ws(M, N, K);
    if (!ws || !aligned(ws, 256) || ws_bytes < w.bytes) return BITLINEAR_EWORKSPACE;
    if (M == 0) return BITLINEAR_OK;
    int8_t* xq = (int8_t*)ws;
    float* eta = (float*)((char*)ws + w.xq);
    int32_t* xsum = w.xsum ? (int32_t*)((char*)ws + w.xq + w.eta) : nullptr;
    void* rest = (char*)ws + w.xq + w.eta + w.xsum;
    hipStream_t s = (hipStream_t)stream;
    clear_hip_error();
    // Up to four tokens on a shape the fused decode kernel takes: each
    // workgroup quantizes the rows itself, one launch (x~ and eta still land
    // in the workspace; no row sums, which no decode kernel reads).
    if (!rmsnorm && K <= kFusedMaxK && forward_path(M, N) == Path::Gemv && gemv_fused_single(M, N, K))
        return launch_gemv_fused_single(make_problem(xq, eta, packed, gamma, N, K, y, nullptr, x), M, s);
    // The quantizer writes the row sums alongside xq, so the contraction
    // need not sum the activation tiles again.
    rc = rmsnorm ? launch_rmsnorm_quantize(x, M, K, xq, eta, xsum, nullptr, s)
                 : launch_quantize(x, M, K, xq, eta, xsum, s);
    if (rc) return rc;
    return run_forward(xq, eta, xsum, packed, gamma, M, N, K, y, nullptr, rest, s);
}

int bitlinear_forward_f32_noalloc(const float* x, const uint8_t* packed, float gamma, int64_t M,
                                  int64_t N, int64_t K, float* y, void* stream) {
    int rc = check_sizes(M, N, K);
    if (rc) return rc;
    if (!x || !packed || !y) return BITLINEAR_EINVAL;
    if (!aligned(x, 16) || !aligned(packed, 16)) return BITLINEAR_EINVAL;
    if (f32_ws(M, N, K).bytes > (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES) return BITLINEAR_EWORKSPACE;
    if (M == 0) return BITLINEAR_OK;
    clear_hip_error();
    void* ws = scratch_for_current_device();
    if (!ws) return BITLINEAR_EHIP;
    // Nothing in the workspace needs a starting value: x~, eta and the row
    // sums are written by the quantizer, split-K partials by every slice
    // before the epilogue reads them.
    return forward_f32_common(x, packed, gamma, M, N, K, y, ws, (size_t)BITLINEAR_NOALLOC_SCRATCH_BYTES,
                              stream, false);
}

int bitlinear_forward_f32(const float* x, const uint8_t* packed, float gamma, int64_t M, int64_t N,
                          int64_t K, float* y, void* ws, size_t ws_bytes, void* stream) {
    return forward_f32_common(x, packed, gamma, M, N, K, y, ws, ws_bytes, stream, false);
}

int bitlinear_forward_rmsnorm_f32(const float* x, const uint8_t* packed, float gamma, int64_t M,
                                  int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                                  void* stream) {
    return forward_f32_common(x, packed, gamma, M, N, K, y, ws, ws_bytes, stream, true);
}

size_t bitlinear_grouped_table_bytes(const bitlinear_problem* problems_host, int32_t count,
                                     int64_t M) {
    PlanHost h;
    if (build_plan(problems_host, count, M, h) != BITLINEAR_OK) return 0;
    return table_layout(count, (int64_t)h.units.size(), (int64_t)h.rows.size(), h.kernel, M).bytes;
}

int bitlinear_grouped_plan_init(const bitlinear_problem* problems_host, int32_t count, int64_t M,
                                void* table, size_t table_bytes, bitlinear_grouped_plan* plan,
                                void* stream) {
    if (!plan) return BITLINEAR_EINVAL;
    PlanHost h;
    int rc = build_plan(problems_host, count, M, h);
    if (rc) return rc;
    const TableLayout L = table_layout(count, (int64_t)h.units.size(), (int64_t)h.rows.size(), h.kernel, M);
    if (!table || !aligned(table, 256) || table_bytes < L.bytes) return BITLINEAR_EWORKSPACE;
    std::vector<uint8_t> host(L.part_off, 0);   // the partials need no initial value
    std::memcpy(host.data() + L.problems_off, h.problems.data(), h.problems.size() * sizeof(Problem));
    std::memcpy(host.data() + L.units_off, h.units.data(), h.units.size() * sizeof(Unit));
    if (!h.rows.empty())
        std::memcpy(host.data() + L.rows_off, h.rows.data(), h.rows.size() * sizeof(QuantRow));
    hipStream_t s = (hipStream_t)stream;
    clear_hip_error();
    BL_HIP_CHECK(hipMemcpyAsync(table, host.data(), L.part_off, hipMemcpyHostToDevice, s));
    BL_HIP_CHECK(hipStreamSynchronize(s));
    int max_K = 0;
    for (const Problem& p : h.problems) max_K = p.K > max_K ? p.K : max_K;
    plan->table = table;
    plan->table_bytes = L.bytes;
    plan->units = (int64_t)h.units.size();
    plan->quant_rows = (int64_t)h.rows.size();
    plan->count = count;
    plan->M = (int32_t)M;
    plan->kernel = h.kernel;
    plan->max_K = max_K;
    return BITLINEAR_OK;
}

int bitlinear_forward_grouped(const bitlinear_grouped_plan* plan, void* stream) {
    if (!plan || !plan->table || plan->count <= 0 || plan->M < 0) return BITLINEAR_EINVAL;
    if (plan->M == 0) return BITLINEAR_OK;
    if (plan->kernel < kPlanGemv || plan->kernel > kPlanLast) return BITLINEAR_EINVAL;
    const TableLayout L = table_layout(plan->count, plan->units, plan->quant_rows, plan->kernel, plan->M);
    if (plan->table_bytes < L.bytes) return BITLINEAR_EINVAL;
    const char* base = (const char*)plan->table;
    const Problem* problems = (const Problem*)(base + L.problems_off);
    const Unit* units = (const Unit*)(base + L.units_off);
    const QuantRow* rows = (const QuantRow*)(base + L.rows_off);
    hipStream_t s = (hipStream_t)stream;
    clear_hip_error();
    int rc = BITLINEAR_OK;
    if (plan->quant_rows)
        rc = launch_quantize_grouped(rows, plan->quant_rows,
                                     plan->kernel != kPlanGemv && plan->kernel != kPlanGemvSplit, s);
    if (rc) return rc;
    switch (plan->kernel) {
        case kPlanGemv: return launch_gemv_grouped(problems, units, plan->units, plan->M, nullptr, s);
        case kPlanGemvFused: return launch_gemv_fused(problems, units, plan->units, plan->M, plan->max_K, s);
        case kPlanGemvSplit:
            return launch_gemv_grouped(problems, units, plan->units, plan->M,
                                       reinterpret_cast<int32_t*>(static_cast<char*>(plan->table) + L.part_off), s);
        case kPlanSkinny: return launch_skinny_grouped(problems, units, plan->units, plan->M, nullptr, s);
        case kPlanSkinnySplit:
            return launch_skinny_grouped(problems, units, plan->units, plan->M,
                                         reinterpret_cast<int32_t*>(static_cast<char*>(plan->table) + L.part_off), s);
        case kPlanGemmSplit:
            return launch_gemm_grouped(problems, units, plan->units, plan->M, true,
                                       reinterpret_cast<int32_t*>(static_cast<char*>(plan->table) + L.part_off), s);
        case kPlanGemmSmall: return launch_gemm_grouped(problems, units, plan->units, plan->M, true, nullptr, s);
        case kPlanBase3:
        case kPlanBase3Split: {
            // no slice is longer than the longest K or than the LDS arrangement allows
            int64_t max_kb = base3_max_slice_kb(plan->M);
            if (ceil_div(plan->max_K, kBase3BlockK) < max_kb) max_kb = ceil_div(plan->max_K, kBase3BlockK);
            return launch_base3_grouped(problems, units, plan->units, plan->M, max_kb,
                                        plan->kernel == kPlanBase3Split
                                            ? reinterpret_cast<int32_t*>(static_cast<char*>(plan->table) + L.part_off)
                                            : nullptr,
                                        s);
        }
        default: return launch_gemm_grouped(problems, units, plan->units, plan->M, false, nullptr, s);
    }
}

}  // extern "C"
