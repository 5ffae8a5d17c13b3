// xcd.h -- block index -> work item map for the chip's eight XCDs.
#pragma once

namespace bl {

// Workgroups are dispatched to the 8 XCDs round robin (block i -> XCD i % 8),
// and each XCD has its own L2.  Renumber work items so that XCD x gets a
// contiguous range of them: with N-tiles fastest, an XCD then owns whole rows
// of token tiles -- each A tile is fetched into one L2 only -- and, for a
// stack of problems in one launch (the batch flattened into the block index,
// problem-major), whole problems: a layer's tiles share its codes and weights
// in one L2 instead of fetching them into up to eight.  XCD x takes
// items [start_x, start_x + count_x) with count_x = ceil((T - x) / 8), the
// number of block indices i < T with i % 8 == x, so the map is one-to-one
// for any T.
__device__ __forceinline__ int xcd_tile(int bid, int tiles) {
    constexpr int kXcds = 8;
    const int x = bid % kXcds, i = bid / kXcds;
    const int q = tiles / kXcds, r = tiles % kXcds;
    return x * q + min(x, r) + i;
}

}  // namespace bl
