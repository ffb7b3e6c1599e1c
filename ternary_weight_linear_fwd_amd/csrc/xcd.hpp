// xcd.hpp -- workgroup-to-work mapping across the XCDs of the chip.
#pragma once
#include <stdint.h>

namespace bl {

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8), each with its own L2.  This permutation hands each XCD a
// contiguous run of the T work items, in order, so that the items an XCD
// runs at one time are neighbours: their operands share its L2 and their
// outputs and weight streams are adjacent in memory.  A bijection of
// [0, T) for any T; only performance depends on the dispatch order.
__device__ inline uint32_t xcd_contiguous(uint32_t b, uint32_t T) {
    constexpr uint32_t X = 8;
    const uint32_t xcd = b % X, slot = b / X, q = T / X, r = T % X;
    return xcd * q + (xcd < r ? xcd : r) + slot;
}

}  // namespace bl
