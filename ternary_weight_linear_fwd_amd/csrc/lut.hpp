// lut.hpp -- compact base-3 weight format and the lookup-table decode
// contraction (lut.hip); the matrix-core decode of the base-3 layout
// (base3.hip).
#pragma once
#include "kernels.hpp"

namespace bl {

// Weight formats the lookup-table contraction reads.
constexpr int kFormat2Bit = 0;   // the 2-bit device layout
constexpr int kFormatBase3 = 1;  // the base-3 device layout

// Base-3 device layout: 64-row groups x blocks of 80 k, 1024 bytes per block
// (16 bytes per row; byte p holds k = 80b + 5p + j as the base-3 digit of 3^j
// of v, stored in the fraction form q = ceil(256 v / 243)).
constexpr int kBase3BlockK = 80;
__host__ __device__ inline uint32_t base3_fraction_byte(uint32_t v) { return (256u * v + 242u) / 243u; }
__host__ __device__ inline uint32_t base3_canonical_byte(uint32_t q) { return (243u * q) >> 8; }
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

// Matrix-core contraction of the base-3 layout (base3.hip): up to
// kBase3MaxTokens tokens per pass over the weights; split-K partial sums in
// the workspace.
constexpr int kBase3MaxTokens = 8;
// 256-row blocks one grouped work unit runs (unsplit problems): fewer for
// more tokens, whose per-block outputs the unit stages in LDS (at most 8 KB).
constexpr int base3_unit_blocks(int64_t M) { return M <= 2 ? 4 : (M <= 4 ? 2 : 1); }
size_t base3_ws_bytes(int64_t M, int64_t N, int64_t K);
int launch_base3(const Problem& p, int64_t M, void* ws, hipStream_t stream);
// Longest K-slice (80-k blocks) one workgroup arranges in LDS for mc tokens.
int64_t base3_max_slice_kb(int64_t mc);
// Grouped (M <= kBase3MaxTokens): problem p's units are its 256-row blocks,
// each cut into p.slices K-slices (consecutive units; p.Kb holds the 80-k
// block count); max_slice_kb bounds every slice's length.  With any slices >
// 1, partial holds nunits * M * 256 int32 and a second launch adds the
// slices and dequantizes.
int launch_base3_grouped(const Problem* problems, const Unit* units, int64_t nunits, int64_t M,
                         int64_t max_slice_kb, int32_t* partial, hipStream_t stream);

}  // namespace bl
