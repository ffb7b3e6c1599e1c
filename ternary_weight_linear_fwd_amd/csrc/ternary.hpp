// ternary.hpp -- ternarization of one latent weight, shared by the 2-bit and
// base-3 packers.
//
// [P1] "1. Absmean Weight Quantization" and the WeightQuantizerSTE listing:
// W~ = Clip(Round(W / gamma), -1, +1), an IEEE division and round half to even.
#pragma once
#include "common.hpp"

namespace bl {

// Code (= digit) of one ternarized weight: w + 1 in {0, 1, 2}.
__device__ inline uint32_t ternary_code(float w, float gamma) {
    const float t = __fdiv_rn(w, gamma);
    const float r = fminf(fmaxf(rintf(t), -1.0f), 1.0f);
    return (uint32_t)((int)r + 1);
}

}  // namespace bl
