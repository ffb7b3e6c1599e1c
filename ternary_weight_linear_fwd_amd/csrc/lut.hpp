// lut.hpp -- compact base-3 weight format and the lookup-table decode
// contraction (lut.hip).
#pragma once
#include "kernels.hpp"

namespace bl {

// Weight formats the lookup-table contraction reads.
constexpr int kFormat2Bit = 0;   // the 2-bit device layout
constexpr int kFormatBase3 = 1;  // the base-3 device layout

// Base-3 device layout: 64-row groups x blocks of 80 k, 1024 bytes per block
// (16 bytes per row; byte p holds k = 80b + 5p + j as the base-3 digit of 3^j).
constexpr int kBase3BlockK = 80;
size_t packed3_bytes(int64_t N, int64_t K);

int launch_pack_weights3(const float* W, int64_t N, int64_t K, uint8_t* packed3, float* gamma_dev,
                         void* ws, hipStream_t stream);
int launch_pack_ternary3(const int8_t* Wt, int64_t N, int64_t K, uint8_t* packed3, int32_t* bad,
                         hipStream_t stream);
int launch_unpack3(const uint8_t* packed3, int64_t N, int64_t K, int8_t* Wt, int32_t* bad,
                   hipStream_t stream);

// The workspace the lookup-table contraction needs (split-K partial sums).
size_t lut_ws_bytes(int64_t M, int64_t N, int64_t K, int format);
// p.packed points at the format's device layout; p.Kb is ignored.
int launch_lut(const Problem& p, int64_t M, int format, void* ws, hipStream_t stream);

}  // namespace bl
