// gemm_common.hpp -- tile scheduling shared by the quantized GEMMs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

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

namespace dmpq {

// ---------------------------------------------------------------------------
// Epilogue staging.  A wave's output tile is 128 x 128; it is written out in
// two bands of 64 rows.  The accumulators (transposed MFMA layout: lane =
// row, 4 consecutive columns per register group) are converted and written
// into a per-wave LDS band, which is then read back row-contiguous so that
// every global store instruction writes whole rows, 16 bytes per lane.
// ---------------------------------------------------------------------------
constexpr int kEpiRows = 64;
template <int ESIZE>
struct EpiBand {
    static constexpr int ROW_BYTES = 128 * ESIZE;      // 128 output columns
    static constexpr int STRIDE = ROW_BYTES + 16;      // padded LDS row
    static constexpr int BYTES = kEpiRows * STRIDE;    // per-wave LDS band
    static constexpr int LANES_PER_ROW = ROW_BYTES / 16;
    static constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
};

// Copy one wave's LDS band (kEpiRows x 128 values of ESIZE bytes) to y at
// (row0, col0), clipping to M x N.  vec: rows of y are 16-byte aligned.
template <int ESIZE>
__device__ __forceinline__ void epi_band_to_global(const uint8_t *band, void *y, int64_t M,
                                                   int64_t N, int64_t row0, int64_t col0,
                                                   int lane, bool vec) {
    using B = EpiBand<ESIZE>;
    constexpr int PER = 16 / ESIZE;  // values per lane per pass
    const int chunk = lane % B::LANES_PER_ROW;
    const int64_t col = col0 + chunk * PER;
#pragma unroll 4
    for (int p = 0; p < kEpiRows / B::ROWS_PER_PASS; p++) {
        const int r = p * B::ROWS_PER_PASS + lane / B::LANES_PER_ROW;
        const int64_t row = row0 + r;
        const uint4 v = *reinterpret_cast<const uint4 *>(band + r * B::STRIDE + chunk * 16);
        if (row >= M || col >= N) continue;
        uint8_t *dst = static_cast<uint8_t *>(y) + (row * N + col) * ESIZE;
        if (vec && col + PER <= N) {
            // streaming store: every tile of a launch finishes at about the same
            // time, and the burst of outputs drains faster without L2 allocation
            store_nt16(dst, v);
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < PER; e++) {
                if (col + e >= N) break;
                if constexpr (ESIZE == 4)
                    reinterpret_cast<uint32_t *>(dst)[e] = w[e];
                else
                    reinterpret_cast<uint16_t *>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

}  // namespace dmpq
