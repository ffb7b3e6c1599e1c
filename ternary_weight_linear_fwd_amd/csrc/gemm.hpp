// gemm.hpp -- the single-problem prefill contraction (gemm.hip) and the
// activation row sums it takes.
#pragma once
#include "kernels.hpp"

namespace bl {

// Workspace of a prefill contraction: the row sums xsum [M] when the caller
// has none, or the int32 partial sums [S][M][N] when the K loop is split.
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K);

// xsum[m] = sum_k xq[m][k] (int32, wrapping), queued on the stream.
int launch_rowsum(const int8_t* xq, int64_t M, int64_t K, int32_t* xsum, hipStream_t stream);

// Prefill contraction (M > 64) with the fused dequant epilogue, given the
// exact row sums xsum[m] = sum_k xq[m][k] (from launch_rowsum or the
// activation quantizer).  ws holds gemm_ws_bytes(M, N, K) bytes and does
// not overlap xsum.
int launch_gemm_xsum(const Problem& p, int64_t M, const int32_t* xsum, void* ws, hipStream_t stream);

// Compute units of the current device (cached per device; 256 if unknown).
int device_cus();

// Whether this kernel, rather than the streaming MFMA decode kernel, should
// contract M <= 64 tokens against N rows.
bool gemm_beats_skinny(int64_t M, int64_t N);

// The same without row sums; ws holds gemm_ws_bytes(M, N, K) bytes.
int launch_gemm(const Problem& p, int64_t M, void* ws, hipStream_t stream);

}  // namespace bl
