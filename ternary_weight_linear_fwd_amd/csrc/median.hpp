// median.hpp -- the absmedian weight scale (median.hip).
#pragma once
#include "kernels.hpp"

namespace bl {

size_t median_ws_bytes();

// gamma = clamp(median of |W|, 1e-5) into gamma_dev (may be null) and into the
// workspace float *gamma_ws points at afterwards; then the 2-bit packing.
int launch_absmedian_gamma(const float* W, int64_t N, int64_t K, float* gamma_dev, void* ws,
                           const float** gamma_ws, hipStream_t stream);
int launch_pack_weights_absmedian(const float* W, int64_t N, int64_t K, uint8_t* packed,
                                  float* gamma_dev, void* ws, const float** gamma_ws,
                                  hipStream_t stream);

}  // namespace bl
