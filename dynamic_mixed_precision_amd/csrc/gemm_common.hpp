// gemm_common.hpp -- tile scheduling shared by the quantized GEMMs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmpq {

// Map a 1-D workgroup id onto an (m, n) output tile.
// 1. XCD-aware: the dispatcher deals workgroups round-robin to the 8 XCDs
//    (id % 8), each with its own L2.  Renumber so that each XCD receives a
//    contiguous range of logical ids (the ids beyond the last multiple of 8
//    keep their number).
// 2. Grouped order: consecutive logical ids walk down a band of `group_m`
//    tile rows before moving right, so the A rows and W columns one XCD is
//    working on at a time stay few and L2-resident.
struct TileCoord {
    unsigned m, n;
};

__device__ __forceinline__ TileCoord tile_of(unsigned bid, unsigned nwg, unsigned tiles_m,
                                             unsigned tiles_n, unsigned group_m) {
    const unsigned full = nwg & ~7u;
    unsigned pid = bid;
    if (bid < full) pid = (bid & 7u) * (full >> 3) + (bid >> 3);
    const unsigned per_group = group_m * tiles_n;
    const unsigned g = pid / per_group;
    const unsigned first_m = g * group_m;
    const unsigned rows = min(tiles_m - first_m, group_m);
    const unsigned in_group = pid - g * per_group;
    return TileCoord{first_m + in_group % rows, in_group / rows};
}

}  // namespace dmpq
