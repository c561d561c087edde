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

typedef float v16f __attribute__((ext_vector_type(16)));

// fp32 accumulators of a 128 x 128 wave tile in the transposed MFMA layout
// (lane l owns row l % 32 of A-subtile i and four consecutive output columns
// 8g + 4*(l/32) + 0..3 of W-subtile j per register group g) -> y =
// (acc * gA) * gW in fp32 or bf16, staged per wave through LDS in two 64-row
// bands and stored row-contiguous.  The caller guarantees that no other wave
// still reads this wave's band region.
template <int OUT>
__device__ __forceinline__ void f32_band_epilogue(v16f (&acc)[4][4], uint8_t *lds, float gA,
                                                  float gW, int64_t M, int64_t N, int64_t m0,
                                                  int64_t n0, int wave, int wm, int wn, int lane,
                                                  void *y) {
    constexpr int ES = OUT == 1 ? 2 : 4;
    using Band = EpiBand<ES>;
    const int lm = lane & 31, lh = lane >> 5;
    uint8_t *band = lds + wave * Band::BYTES;
    const bool vec = ((N * ES) & 15) == 0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            const int i = 2 * h + ii;
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    uint8_t *dst = band + (ii * 32 + lm) * Band::STRIDE + (j * 32 + 8 * g + 4 * lh) * ES;
                    float v4[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) v4[e] = (acc[i][j][4 * g + e] * gA) * gW;
                    if constexpr (OUT == 0)
                        *reinterpret_cast<float4 *>(dst) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                    else
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(cvt_pk_bf16(v4[0], v4[1]), cvt_pk_bf16(v4[2], v4[3]));
                }
            }
        }
        epi_band_to_global<ES>(band, y, M, N, m0 + wm * 128 + h * 64, n0 + wn * 128, lane, vec);
    }
}

}  // namespace dmpq
