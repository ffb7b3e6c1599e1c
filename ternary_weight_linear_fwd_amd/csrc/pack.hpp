// pack.hpp -- pieces of the weight packer (pack.hip) shared with the base-3
// packer (lut.hip).
#pragma once
#include "kernels.hpp"

namespace bl {

// gamma of W into gamma_dev (may be null) and into the workspace float that
// follows the kGammaBins bins; the workspace is gamma_ws_bytes() long.
int launch_gamma(const float* W, int64_t N, int64_t K, float* gamma_dev, void* ws,
                 hipStream_t stream);

// Ternarize W with the scale at gamma_dev (device) and write the 2-bit layout.
int launch_ternarize_pack(const float* W, int64_t N, int64_t K, const float* gamma_dev,
                          uint8_t* packed, hipStream_t stream);

// *p = 0, queued on the stream.
int launch_zero_i32(int32_t* p, hipStream_t stream);

}  // namespace bl
