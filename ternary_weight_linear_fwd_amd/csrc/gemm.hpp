// gemm.hpp -- the prefill contraction (gemm.hip) with row sums supplied by
// the caller.
#pragma once
#include "kernels.hpp"

namespace bl {

// As launch_gemm, with xsum[m] = sum_k xq[m][k] (exact, as the activation
// quantizer writes it) read instead of summed from the activation tiles.
// xsum null: launch_gemm.
int launch_gemm_xsum(const Problem& p, int64_t M, const int32_t* xsum, hipStream_t stream);

}  // namespace bl
