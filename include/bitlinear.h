/*
 * bitlinear.h -- C ABI of the BitNet b1.58 BitLinear forward pass for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (cited by page title and section):
 *  [P1] "BitNet b1.58 & 1-Bit LLMs in Production: Ternary Quantization,
 *       MatMul-Free Kernels, and Edge AI Silicon Deployment"
 *  [P2] "1-Bit Large Language Models and BitNet b1.58: How Ternary Weights and
 *       Additive Kernels Eliminate Matrix Multiplications"
 *  [P4] "BitNet b1.58 & 1-Bit LLM Architectures: Eliminating Matrix
 *       Multiplication and Running 70B Models on CPU in 2026"
 *  [P5] "BitNet b1.58: Ternary Weight LLMs That Eliminate Matrix
 *       Multiplication"
 *
 *   eta[m]   = max(max_k |x[m][k]|, 1e-5)                       per token row
 *   xq[m][k] = clamp(rne((x[m][k] * 127) / eta[m]), -128, 127)   int8
 *   gamma    = max(mean |W|, 1e-5)   (exact mean, rounded once to float32)
 *   Wt[n][k] = clamp(rne(W[n][k] / gamma), -1, 1)                 ternary
 *   y_int    = sum_{Wt=+1} xq - sum_{Wt=-1} xq                    int32
 *   y[m][n]  = float(y_int[m][n]) * ((eta[m] * gamma) / 127)      float32
 * All float steps are single IEEE float32 operations in the order written
 * (no fused multiply-add, correctly rounded division, round half to even).
 *
 * Conventions shared by every call
 *  - Matrices are dense and row-major: x, xq are [M][K]; W, Wt are [N][K]
 *    (output features by input features, as nn.Linear stores them); y and
 *    y_int are [M][N].
 *  - Every pointer is a device pointer (HIP device memory), unless its name
 *    ends in _host.  The caller allocates and frees every buffer; the library
 *    never allocates device memory, keeps no state between calls and is
 *    re-entrant.  Buffers must stay valid until the work queued on `stream`
 *    has finished.
 *  - `stream` is a hipStream_t (NULL is the default stream).  Every call only
 *    queues work on it and returns, except where a call says it synchronizes.
 *  - K must be a multiple of 16 and at most BITLINEAR_MAX_K.  M may be 0
 *    (nothing is queued).  N, K >= 1.
 *  - Inputs must be finite; NaN or Inf give unspecified (but bounded) output.
 *  - Arguments are validated before anything is queued: on a non-zero return
 *    nothing has been written.
 *
 * Packed weight layout ("device layout")
 *   A bijection of the canonical 2-bit format of [P1] "Production Deployment
 *   Standards for Edge Systems Engineers" item 1 and [P5] "Kernel
 *   Implementation: The Lookup Table Approach": codes 00 = -1, 01 = 0,
 *   10 = +1, four weights per byte; code 11 never occurs.  Rows are grouped by
 *   64 and K is cut into blocks of 64; block (g, b) of 1024 bytes holds, for
 *   each of its 64 rows r in order, 16 bytes = 4 little-endian 32-bit words;
 *   word d covers k = 64b + 16d + 4j + i at bits 8i + 2j .. 8i + 2j + 1
 *   (i = byte, j = field).  Rows past N and k past K hold code 01.
 *   Size: bitlinear_packed_bytes(N, K) = ceil(N/64) * ceil(K/64) * 1024.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-valued call. */
#define BITLINEAR_OK 0
#define BITLINEAR_EINVAL (-1)       /* null pointer, negative or zero size, bad count */
#define BITLINEAR_EUNSUPPORTED (-2) /* K not a multiple of 16, K above BITLINEAR_MAX_K,
                                       or another size beyond 2^31 */

/* Longest reduction (input features K) any call accepts.  Every kernel keeps
 * its int32 partial sums and 32-bit operand offsets exact up to this K (the
 * dot4 decode path keeps one code field scaled by 16: |sum| <= 1016 K < 2^31;
 * a 128-row prefill tile spans 128 K < 2^32 activation bytes); the int32
 * result itself needs only 127 K < 2^31. */
#define BITLINEAR_MAX_K (1 << 21)
#define BITLINEAR_EWORKSPACE (-3)   /* workspace missing or smaller than required */
#define BITLINEAR_EBADCODE (-4)     /* a ternary input outside {-1, 0, 1} */
#define BITLINEAR_EHIP (-5)         /* a HIP runtime call or kernel launch failed */

/* Human-readable name of a status code (static storage; never NULL). */
const char* bitlinear_status_string(int status);

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int bitlinear_abi_version(void);

/* The HIP error behind the most recent BITLINEAR_EHIP returned on this host
 * thread: error name, code and the failing call (static thread-local storage;
 * never NULL). */
const char* bitlinear_last_error(void);

/* Bytes of the packed device layout for an N x K ternary matrix (host only;
 * 0 for invalid sizes). */
size_t bitlinear_packed_bytes(int64_t N, int64_t K);

/* Workspace bytes that bitlinear_pack_weights, bitlinear_forward and
 * bitlinear_forward_f32 need for these sizes (host only; 0 for invalid
 * sizes).  One workspace of this size serves all three; it must be 256-byte
 * aligned. */
size_t bitlinear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * Per-token absmax INT8 activation quantization.
 * [P1] "2. Absmax Dynamic Activation Quantization" (Q_b = 127) and the
 * ActivationQuantizerSTE listing of "Production PyTorch Implementation:
 * BitLinear b1.58 Layer"; [P4] "Activation Quantization: 8-Bit Absmax
 * Scaling"; [P2] "2. Absmax Activation Quantization" (per token).
 *   x    [M][K] float32 (in)
 *   xq   [M][K] int8    (out)
 *   eta  [M]    float32 (out)
 *   xsum [M]    int32   (out, may be NULL): sum over k of xq[m][k] (int32,
 *        wrapping), the row sums bitlinear_forward_xsum takes
 */
int bitlinear_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                           int32_t* xsum, void* stream);

/*
 * RMSNorm without affine parameters, then the per-token absmax INT8
 * quantization of the normalized rows, in one pass over x.
 * [P1] pipeline box 1 ("RMSNorm") and step 1 of BitLinear158.forward in
 * "Production PyTorch Implementation: BitLinear b1.58 Layer" (norm =
 * rsqrt(mean(x^2) + 1e-6), x_norm = x * norm); [P1] "2. Absmax Dynamic
 * Activation Quantization" (normalization without affine parameters before
 * the quantizer); [P2] "2. Absmax Activation Quantization".
 *   ms[m]   = the exact mean over k of x[m][k]^2, rounded once to float32
 *   norm    = 1 / sqrt(ms[m] + 1e-6)  (IEEE float32 add, square root, division)
 *   x_norm  = x * norm (float32); eta, xq, xsum as bitlinear_quantize_act
 *             computes them from x_norm
 *   x    [M][K] float32 (in)        xq   [M][K] int8 (out)
 *   eta  [M] float32 (out)          xsum [M] int32 (out, may be NULL)
 *   ms   [M] float32 (out, may be NULL)
 */
int bitlinear_rmsnorm_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                                   int32_t* xsum, float* ms, void* stream);

/*
 * Absmean ternary weight quantization and packing.
 * [P1] "1. Absmean Weight Quantization" and the WeightQuantizerSTE listing;
 * [P2] "1. Absmean Weight Quantization"; [P4] "The Weight Quantization
 * Function: Absmean Scaling"; packing as in the layout note above.
 *   W          [N][K] float32 latent weights (in)
 *   packed     bitlinear_packed_bytes(N, K) bytes (out)
 *   gamma      float32 device scalar (out, may be NULL)
 *   gamma_host float32 host scalar (out, may be NULL); when given, the call
 *              synchronizes `stream` and returns with it written
 *   ws         workspace of bitlinear_workspace_bytes(0, N, K) bytes
 * gamma is the exact mean of |W| over all N*K entries, rounded once to the
 * nearest float32 (ties to even), then clamped below at 1e-5; the result does
 * not depend on summation order.
 */
int bitlinear_pack_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                           float* gamma_host, void* ws, size_t ws_bytes, void* stream);

/*
 * Absmedian variant of bitlinear_pack_weights: gamma is the median of |W| in
 * place of the mean.  [P2] "Scaling Laws and Empirical Benchmarks" (BitNet
 * b1.58 Reloaded's absmedian baseline).  For an even count N*K the median is the mean of the two middle magnitudes, rounded once
 * to the nearest float32 (ties to even); it is clamped below at 1e-5 and the
 * ternarization and 2-bit layout are those of bitlinear_pack_weights.  Same
 * arguments; ws of bitlinear_workspace_bytes(0, N, K) bytes.
 */
int bitlinear_pack_weights_absmedian(const float* W, int64_t N, int64_t K, uint8_t* packed,
                                     float* gamma, float* gamma_host, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * Pack ternary weights that are already in {-1, 0, 1} (e.g. drawn directly,
 * with gamma supplied separately).
 *   Wt     [N][K] int8 (in)
 *   packed bitlinear_packed_bytes(N, K) bytes (out)
 *   bad    int32 device scalar (out, may be NULL): set (on the stream) to the
 *          number of entries outside {-1, 0, 1} (those are packed as 0)
 * Asynchronous; a caller that needs BITLINEAR_EBADCODE reads `bad` after
 * synchronizing.
 */
int bitlinear_pack_ternary(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed,
                           int32_t* bad, void* stream);

/*
 * Unpack the device layout back to ternary int8 [N][K] (round trip, tests).
 *   bad int32 device scalar (out, may be NULL): number of 11 codes found
 *       inside [0, N) x [0, K) (decoded as 0).
 */
int bitlinear_unpack_weights(const uint8_t* packed, int64_t N, int64_t K, int8_t* Wt,
                             int32_t* bad, void* stream);

/*
 * BitLinear forward from quantized activations: the multiplication-free
 * ternary contraction and the fused dequantization.
 * [P1] "The MatMul-Free Breakthrough" and pipeline boxes 4-5; [P2] "3.
 * Additive Integer Accumulation"; [P5] "The Arithmetic Collapse" and the
 * bitlinear_forward listing.
 *   xq     [M][K] int8   (in)
 *   eta    [M]    float32 (in)
 *   packed device layout of the [N][K] ternary matrix (in)
 *   gamma  the matrix's scale (by value)
 *   y      [M][N] float32 (out)
 *   y_int  [M][N] int32   (out, may be NULL): the exact integer sums
 *   ws     workspace of bitlinear_workspace_bytes(M, N, K) bytes, 256-byte
 *          aligned: split-K partial sums (decode kernels, and the tiled
 *          kernel when its 32 x 128 tiles leave CUs idle over a long K), or
 *          room for the activation row sums of the tiled kernel
 * Kernel by size: M <= 4 the dot4 GEMV (with a short K loop per
 * 64-row group: one workgroup per group whose wavefronts split K and add
 * their sums in LDS; otherwise K split over workgroups, with partial sums
 * in ws and a second launch); 4 < M <= 16 the streaming MFMA kernel; M > 16
 * the tiled int8-MFMA kernel (its K loop split over several workgroups per
 * tile when few tiles would leave CUs idle).
 */
int bitlinear_forward(const int8_t* xq, const float* eta, const uint8_t* packed, float gamma,
                      int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * bitlinear_forward with the activation row sums supplied: the same result,
 * bit for bit, when xsum is right.  The tiled contraction (see above) of
 * [P2] "3. Additive Integer Accumulation" runs on the stored weight codes
 * c = w + 1 in {0, 1, 2}: sum_k xq w = sum_k xq c - sum_k xq, so it needs
 * each row's sum; the quantizer produces those sums in the same pass that
 * writes xq, and passing them on spares the contraction summing its
 * activation tiles again.
 *   xsum [M] int32 (in): xsum[m] = sum over k < K of xq[m][k], exactly as
 *        bitlinear_quantize_act or bitlinear_rmsnorm_quantize_act write it.
 *        Not checked: a wrong row sum shifts that row's y_int by the error.
 *        The decode kernels (dot4 and streaming MFMA) do not read it.
 *        It must not overlap ws.
 *   other arguments, workspace and errors as bitlinear_forward.
 */
int bitlinear_forward_xsum(const int8_t* xq, const float* eta, const int32_t* xsum,
                           const uint8_t* packed, float gamma, int64_t M, int64_t N, int64_t K,
                           float* y, int32_t* y_int, void* ws, size_t ws_bytes, void* stream);

/*
 * Fused forward from float32 activations: quantize (into the workspace, with
 * the row sums for bitlinear_forward_xsum), contract, dequantize.  Same
 * arguments as above; ws is required.  At up to four tokens, on the shapes
 * where bitlinear_forward takes the one-workgroup-per-row-group dot4 kernel
 * (and K <= 16384), that kernel quantizes the rows itself in one launch; x~
 * and eta still land in the workspace, the row sums do not.
 * [P1] BitLinear158.forward steps 2, 4 and 5.
 */
int bitlinear_forward_f32(const float* x, const uint8_t* packed, float gamma, int64_t M,
                          int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Allocation-free bitlinear_forward_f32, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same kernels and the same result bits as
 * bitlinear_forward_f32; its workspace is a fixed device array inside the
 * library, BITLINEAR_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library
 * runs on holds until the process ends.  The first call on a device looks up
 * that array's address with the device current; no call allocates.
 *   x, packed, gamma, M, N, K, y, stream as bitlinear_forward_f32.
 * Returns BITLINEAR_EWORKSPACE, before anything is queued, for sizes whose
 * bitlinear_workspace_bytes(M, N, K) exceeds the array.  Every call on one GPU
 * shares the array: calls whose execution overlaps on one GPU (several
 * streams, several host threads) race and give undefined results, so
 * serialize them.  Nothing in the array needs a starting value.
 */
#define BITLINEAR_NOALLOC_SCRATCH_BYTES (64 << 20)
int bitlinear_forward_f32_noalloc(const float* x, const uint8_t* packed, float gamma, int64_t M,
                                  int64_t N, int64_t K, float* y, void* stream);

/*
 * Fused forward with the RMSNorm prologue: normalize and quantize (into the
 * workspace), contract, dequantize.  Same arguments and workspace as
 * bitlinear_forward_f32.  [P1] BitLinear158.forward steps 1, 2, 4 and 5.
 */
int bitlinear_forward_rmsnorm_f32(const float* x, const uint8_t* packed, float gamma, int64_t M,
                                  int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * Compact base-3 weights, five per byte (3^5 = 243 <= 256: 1.6 bits per
 * weight against 2).  [P2] the bandwidth paragraph before "Scaling Laws and
 * Empirical Benchmarks" (1.58 bits per parameter under compact ternary
 * packing); [P3] "Common Misconceptions" (log2(3) bits per ternary weight).
 * Canonical byte: v = sum_j (w[5b + j] + 1) * 3^j, pads weight 0.
 * Base-3 device layout ("base-3 layout"): rows grouped by 64, K cut into
 * blocks of 80; block (g, b) of 1024 bytes holds 16 bytes per row in order,
 * byte p of row r being the fraction form q = ceil(256 v / 243) of the
 * canonical byte v of k = 80b + 5p .. 80b + 5p + 4 (v = floor(243 q / 256);
 * floor(3^s q / 256) is v's top s digits, which the decode uses).  Rows past
 * N and k past K hold weight 0 (q = 128).  The 13 byte values that are no
 * fraction form (1, 20, 40, 60, 79, 99, 119, 138, 158, 178, 197, 217, 237)
 * never occur.
 *   bitlinear_packed3_bytes(N, K) = ceil(N/64) * ceil(K/80) * 1024.
 * pack_weights3, pack_ternary3 and unpack_weights3 mirror the 2-bit calls
 * (same gamma, workspace and `bad` conventions; unpack counts bytes that are
 * no fraction form inside [0, N) x [0, K) and decodes them as zero weights).
 */
size_t bitlinear_packed3_bytes(int64_t N, int64_t K);
int bitlinear_pack_weights3(const float* W, int64_t N, int64_t K, uint8_t* packed3, float* gamma,
                            float* gamma_host, void* ws, size_t ws_bytes, void* stream);
int bitlinear_pack_ternary3(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed3, int32_t* bad,
                            void* stream);
int bitlinear_unpack_weights3(const uint8_t* packed3, int64_t N, int64_t K, int8_t* Wt,
                              int32_t* bad, void* stream);

/*
 * Lookup-table forward: the same contraction and dequantization as
 * bitlinear_forward, computed by table lookups instead of additions.
 * [P3] "What Most People Miss" (precomputed outcomes of small activation
 * blocks, looked up by the weights); [P5] "Kernel Implementation: The Lookup
 * Table Approach".  Each weight byte indexes a per-block table of its
 * activation group's partial sums (5 activations in the base-3 layout, 4 in
 * the 2-bit layout).  Any M is accepted; the path is built for decode (small
 * M).  Results are identical to bitlinear_forward's.
 *   format  BITLINEAR_FORMAT_2BIT (packed: device layout) or
 *           BITLINEAR_FORMAT_BASE3 (packed: base-3 layout)
 *   ws      workspace of bitlinear_lut_workspace_bytes(M, N, K, format) bytes
 */
#define BITLINEAR_FORMAT_2BIT 0
#define BITLINEAR_FORMAT_BASE3 1
size_t bitlinear_lut_workspace_bytes(int64_t M, int64_t N, int64_t K, int format);
int bitlinear_forward_lut(const int8_t* xq, const float* eta, const uint8_t* packed, int format,
                          float gamma, int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * Base-3 forward: the contraction and dequantization of bitlinear_forward,
 * read straight from the base-3 layout (1.6 bits per weight) on the matrix
 * cores; results identical to bitlinear_forward's.  [P2] the bandwidth
 * paragraph before "Scaling Laws and Empirical Benchmarks" (compact ternary
 * packing) and "3. Additive Integer Accumulation".  Built for decode: each
 * pass over the weights serves up to 8 tokens, so larger M costs ceil(M/8)
 * passes.
 *   xq      [M][K] int8, 16-byte aligned; eta [M] float32
 *   packed3 base-3 layout of the [N][K] ternary matrix, 16-byte aligned
 *   y       [M][N] float32; y_int [M][N] int32 or NULL
 *   ws      workspace of bitlinear_forward3_workspace_bytes(M, N, K) bytes
 *           (K-split partial sums; 0 bytes needs no workspace), 256-byte aligned
 * Same errors as bitlinear_forward.
 */
size_t bitlinear_forward3_workspace_bytes(int64_t M, int64_t N, int64_t K);
int bitlinear_forward3(const int8_t* xq, const float* eta, const uint8_t* packed3, float gamma,
                       int64_t M, int64_t N, int64_t K, float* y, int32_t* y_int, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * Grouped forward: many independent BitLinear problems of the same token
 * count M in one pass (e.g. every projection of every layer of a decode
 * step).  Planning builds a work table in caller-owned device memory once;
 * each forward then queues at most three kernels: quantize all, contract all,
 * and -- for a plan too small to fill the chip, whose long K loops the
 * planner splits -- add the split partial sums and dequantize.  A plan of up
 * to four tokens too small to fill the chip (one transformer block, say), with
 * every K at most 16384, queues one kernel that quantizes, contracts and
 * dequantizes; it writes xq and eta of problems with x != NULL all the same.
 * A plan of base-3 problems (format BITLINEAR_FORMAT_BASE3, up to 8 tokens)
 * contracts on the base-3 matrix-core kernel of bitlinear_forward3, with the
 * same results.
 */
typedef struct bitlinear_problem {
    const float* x;        /* [M][K] float32, or NULL: xq/eta already hold the quantized rows */
    int8_t* xq;            /* [M][K] int8: written by the quantize stage when x != NULL */
    float* eta;            /* [M] float32: likewise */
    const uint8_t* packed; /* the [N][K] ternary matrix in the layout `format` names */
    float* y;              /* [M][N] float32 output */
    int32_t* y_int;        /* [M][N] int32 output or NULL */
    float gamma;           /* the matrix's scale */
    int32_t N;
    int32_t K;
    int32_t format;        /* layout of packed: BITLINEAR_FORMAT_2BIT (0, the device layout) or
                              BITLINEAR_FORMAT_BASE3 (1, the base-3 layout, up to 8 tokens);
                              one format for every problem of a plan */
} bitlinear_problem;

/* Host-side handle of a plan; plain data owned by the caller. */
typedef struct bitlinear_grouped_plan {
    void* table;           /* device memory holding the work table */
    size_t table_bytes;
    int64_t units;         /* work units of the contraction kernel */
    int64_t quant_rows;    /* rows the quantize stage handles (0: no stage) */
    int32_t count;         /* number of problems */
    int32_t M;             /* tokens per problem */
    int32_t kernel;        /* contraction kernel variant chosen by the planner */
    int32_t max_K;         /* longest K among the problems */
} bitlinear_grouped_plan;

/* Device bytes the work table for these problems needs (host only).  Plans
 * whose work units would leave CUs idle (a single transformer block, say) may
 * split their K loops, and the table then also holds the int32 partial sums:
 * M x 64 x 4 bytes per work unit of the dot4 decode path (up to 4 tokens),
 * M x 256 x 4 bytes per unit past 4 tokens and of base-3 plans (whose K
 * loops also split where one would not fit the kernel's LDS). */
size_t bitlinear_grouped_table_bytes(const bitlinear_problem* problems_host, int32_t count,
                                     int64_t M);

/* Validate the problems, build the work table in `table` (device memory of
 * bitlinear_grouped_table_bytes bytes) and fill *plan.  Synchronizes `stream`
 * (the table is uploaded from a host copy).  Problems may share x, xq and
 * eta buffers only when they also share x. */
int bitlinear_grouped_plan_init(const bitlinear_problem* problems_host, int32_t count, int64_t M,
                                void* table, size_t table_bytes, bitlinear_grouped_plan* plan,
                                void* stream);

/* Queue the grouped forward described by a plan.  Calls with one plan whose
 * execution overlaps (other streams) race on its table's partial sums. */
int bitlinear_forward_grouped(const bitlinear_grouped_plan* plan, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
