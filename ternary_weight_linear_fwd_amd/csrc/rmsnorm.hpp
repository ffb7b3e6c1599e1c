// rmsnorm.hpp -- launcher of the fused RMSNorm + absmax quantizer (rmsnorm.hip).
#pragma once
#include "common.hpp"

namespace bl {

// x [M][K] float32 -> xq [M][K] int8, eta [M], optional xsum [M] and the
// per-row mean of the squares ms [M].  K % 4 == 0, x 16-byte aligned.
int launch_rmsnorm_quantize(const float* x, int64_t M, int64_t K, int8_t* xq, float* eta,
                            int32_t* xsum, float* ms, hipStream_t stream);

}  // namespace bl
