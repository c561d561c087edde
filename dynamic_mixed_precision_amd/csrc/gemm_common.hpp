// gemm_common.hpp -- tile scheduling shared by the quantized GEMMs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "internal.hpp"

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

__device__ __forceinline__ unsigned xcd_order(unsigned bid, unsigned nwg) {
    const unsigned full = nwg & ~7u;
    return bid < full ? (bid & 7u) * (full >> 3) + (bid >> 3) : bid;
}

__device__ __forceinline__ TileCoord tile_at(unsigned pid, unsigned tiles_m, unsigned tiles_n,
                                             unsigned group_m) {
    const unsigned per_group = group_m * tiles_n;
    const unsigned g = pid / per_group;
    const unsigned first_m = g * group_m;
    const unsigned rows = min(tiles_m - first_m, group_m);
    const unsigned in_group = pid - g * per_group;
    return TileCoord{first_m + in_group % rows, in_group / rows};
}

__device__ __forceinline__ TileCoord tile_of(unsigned bid, unsigned nwg, unsigned tiles_m,
                                             unsigned tiles_n, unsigned group_m) {
    return tile_at(xcd_order(bid, nwg), tiles_m, tiles_n, group_m);
}

// A split workgroup of a SplitPlan launch: workgroup j runs the K stages
// [s * nk / splits, (s + 1) * nk / splits) of tail tile full + j / splits,
// s = j % splits.
struct SplitUnit {
    TileCoord tc;
    int kt0, kt1;
};

__device__ __forceinline__ SplitUnit split_unit(const SplitPlan &sp, unsigned tiles_m, unsigned tiles_n,
                                                unsigned group_m) {
    const unsigned j = blockIdx.x;
    const unsigned s = j % sp.splits;
    SplitUnit u;
    u.tc = tile_at(sp.full + j / sp.splits, tiles_m, tiles_n, group_m);
    u.kt0 = (int)((int64_t)s * sp.nk / sp.splits);
    u.kt1 = (int)((int64_t)(s + 1) * sp.nk / sp.splits);
    return u;
}

// Host: the split plan of a launch of `tiles` tiles with nk K stages each.
// The tail is split into as many parts as fit in one wave of kMaxSplitUnits
// workgroups (at most one stage each; 2, 3, 4 or 8 parts); a tail that
// cannot be split at least in two is not split.
inline SplitPlan plan_split(int64_t tiles, int nk, bool enable) {
    SplitPlan p{(unsigned)tiles, 0u, 1u, nk};
    const int64_t tail = tiles % 256;
    if (!enable || tail == 0) return p;
    int64_t S = (int64_t)kMaxSplitUnits / tail;
    if (S > nk) S = nk;
    S = S >= 8 ? 8 : S >= 4 ? 4 : S;  // 2, 3, 4 or 8: the fixup is compiled per count
    if (S < 2) return p;
    p.full = (unsigned)(tiles - tail);
    p.tail = (unsigned)tail;
    p.splits = (unsigned)S;
    return p;
}

// Raw accumulators of one split workgroup: 256 words per thread, as 64
// 16-byte pieces (register group g of MFMA block (i, j) is piece 4(4i+j)+g);
// for each piece the workgroup writes 4 KB contiguously.
template <class AccV>
__device__ __forceinline__ void store_split_partial(const AccV (&acc)[4][4], uint32_t *part, int tid) {
    typedef decltype(acc[0][0][0] + 0) T;
    uint4 *p4 = reinterpret_cast<uint4 *>(part);
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                // copy the elements out first: a bit cast of a vector-element
                // lvalue reads from the vector's base, i.e. element 0
                const T v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
                const T v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
                p4[((i * 4 + j) * 4 + g) * 256 + tid] =
                    make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                               __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3));
            }
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

// Epilogue options (bit flags).  kEpiGelu: GELU(v) = v Phi(v) of the output
// value as a separate bf16 (or fp32) activation op would see it: the GEMM
// result is rounded to the output type first, GELU runs in fp32 and its
// result is rounded again.  kEpiAmax (bf16 output, N % 16 == 0): the maximum
// of |FWHT16(row block)| over the stored bf16 values of the tile -- the next
// layer's NVFP4 tensor-amax term, with the same fp32 butterfly order as the
// quantizer -- is written to the tile's entry of the maxima.
enum { kEpiGelu = 1, kEpiAmax = 2 };

// GELU(v) = v Phi(v) = (v / 2) erfc(-v / sqrt 2) in fp32.  erfc comes from
// the Chebyshev fit published in Numerical Recipes (Press et al., section
// 6.2, "erfcc": erfc(z) = t exp(-z^2 + P(t)), t = 1 / (1 + z/2), z >= 0, and
// 2 - erfc(-x) for x < 0), whose fractional error is below 1.2e-7 for every
// argument.  The fp32 evaluation adds a few ulp plus the rounding of the
// exponent, a relative error of about v^2 * 1.2e-7 in erfc's tail.  About 20
// VALU operations, no branches: the library erfcf costs several times that.
__device__ __forceinline__ float gelu_f32(float v) {
    const float x = v * -0.70710678118654752f;
    const float z = __builtin_fabsf(x);
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, z, 1.0f));
    float p = 0.17087277f;
    p = __builtin_fmaf(t, p, -0.82215223f);
    p = __builtin_fmaf(t, p, 1.48851587f);
    p = __builtin_fmaf(t, p, -1.13520398f);
    p = __builtin_fmaf(t, p, 0.27886807f);
    p = __builtin_fmaf(t, p, -0.18628806f);
    p = __builtin_fmaf(t, p, 0.09678418f);
    p = __builtin_fmaf(t, p, 0.37409196f);
    p = __builtin_fmaf(t, p, 1.00002368f);
    p = __builtin_fmaf(t, p, -1.26551223f);
    const float e = t * __builtin_amdgcn_exp2f(__builtin_fmaf(-z, z, p) * 1.44269504088896341f);
    return 0.5f * v * (x >= 0.0f ? e : 2.0f - e);
}

// Copy one wave's LDS band (ROWS x 128 values of ESIZE bytes) to y at
// (row0, col0), clipping to M x N.  vec: rows of y are 16-byte aligned.
// kEpiGelu: each value passes through GELU on its way out.  kEpiAmax (bf16
// only): the two lanes holding one 16-block finish its Hadamard (stages 1,
// 2, 4 in-lane, stage 8 across the lane pair, then * 1/4) and the lane's max
// |value| over valid blocks is returned.
template <int ESIZE, int EPI = 0, int ROWS = kEpiRows>
__device__ __forceinline__ float epi_band_to_global(const uint8_t *band, void *y, int64_t M,
                                                    int64_t N, int64_t row0, int64_t col0,
                                                    int lane, bool vec) {
    using B = EpiBand<ESIZE>;
    constexpr int PER = 16 / ESIZE;  // values per lane per pass
    constexpr bool AMAX = (EPI & kEpiAmax) != 0;
    static_assert(!AMAX || ESIZE == 2, "the fused amax reads bf16 outputs");
    const int chunk = lane % B::LANES_PER_ROW;
    const int64_t col = col0 + chunk * PER;
    float amax = 0.0f;
#pragma unroll 4
    for (int p = 0; p < ROWS / B::ROWS_PER_PASS; p++) {
        const int r = p * B::ROWS_PER_PASS + lane / B::LANES_PER_ROW;
        const int64_t row = row0 + r;
        uint4 v = *reinterpret_cast<const uint4 *>(band + r * B::STRIDE + chunk * 16);
        if constexpr ((EPI & kEpiGelu) != 0) {
            if constexpr (ESIZE == 2) {
                v.x = cvt_pk_bf16(gelu_f32(bf16_lo(v.x)), gelu_f32(bf16_hi(v.x)));
                v.y = cvt_pk_bf16(gelu_f32(bf16_lo(v.y)), gelu_f32(bf16_hi(v.y)));
                v.z = cvt_pk_bf16(gelu_f32(bf16_lo(v.z)), gelu_f32(bf16_hi(v.z)));
                v.w = cvt_pk_bf16(gelu_f32(bf16_lo(v.w)), gelu_f32(bf16_hi(v.w)));
            } else {
                v.x = __float_as_uint(gelu_f32(__uint_as_float(v.x)));
                v.y = __float_as_uint(gelu_f32(__uint_as_float(v.y)));
                v.z = __float_as_uint(gelu_f32(__uint_as_float(v.z)));
                v.w = __float_as_uint(gelu_f32(__uint_as_float(v.w)));
            }
        }
        if constexpr (AMAX) {
            float f[8];
            f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
            f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
#pragma unroll
            for (int h = 1; h < 8; h <<= 1)
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if ((i & h) == 0) {
                        const float a = f[i], b = f[i + h];
                        f[i] = a + b;
                        f[i + h] = a - b;
                    }
            const bool lo = (chunk & 1) == 0;  // this lane holds elements 0..7 of the block
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                // the partner lane's value: DPP quad_perm [1, 0, 3, 2] swaps
                // lanes 2k and 2k+1 inside the VALU (no LDS round trip)
                const float o = __int_as_float(
                    __builtin_amdgcn_mov_dpp(__float_as_int(f[i]), 0xB1, 0xF, 0xF, false));
                const float w = lo ? f[i] + o : o - f[i];
                m = fmaxf(m, __builtin_fabsf(w * 0.25f));
            }
            if (row < M && col < N) amax = fmaxf(amax, m);
        }
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
    return amax;
}

typedef float v16f __attribute__((ext_vector_type(16)));

// The fused amax of a 256 x 256 tile: every wave's maximum, combined through
// LDS, written by one lane to *slot (the tile's own entry).  Called by all
// four waves.
__device__ __forceinline__ void epi_tile_amax(float m, int wave, int lane, float *slot) {
    __shared__ float red[4];
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (wave == 0 && lane == 0) *slot = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Output scaling of fp32 accumulators: y = (acc * gA) * gW.
struct EpiScaleF32 {
    float gA, gW;
    __device__ __forceinline__ void row(int64_t) {}
    __device__ __forceinline__ float operator()(float a, int, int, int) const { return (a * gA) * gW; }
};

// Generic band epilogue: accumulators in the transposed MFMA layout (lane l
// owns row l % 32 of A-subtile i and four consecutive output columns
// 8g + 4*(l/32) + 0..3 of W-subtile j per register group g) -> sc (scaling)
// -> (GELU) -> fp32 or bf16 into the per-wave LDS band, then row-contiguous
// stores (and the fused amax).  The caller guarantees that no other wave
// still reads this wave's band region.
template <int OUT, int EPI, class AccV, class Scale>
__device__ __forceinline__ void band_epilogue(AccV (&acc)[4][4], Scale &sc, uint8_t *lds, int64_t M,
                                              int64_t N, int64_t m0, int64_t n0, int wave, int wm,
                                              int wn, int lane, void *y, float *slot) {
    constexpr int ES = OUT == 1 ? 2 : 4;
    constexpr bool AMAX = (EPI & kEpiAmax) != 0;
    static_assert(!AMAX || OUT == 1, "the fused amax needs bf16 output");
    using Band = EpiBand<ES>;
    const int lm = lane & 31, lh = lane >> 5;
    uint8_t *band = lds + wave * Band::BYTES;
    const bool vec = ((N * ES) & 15) == 0;
    float amax = 0.0f;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int ii = 0; ii < 2; ii++) {
            const int i = 2 * h + ii;
            sc.row(m0 + wm * 128 + i * 32 + lm);
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    uint8_t *dst = band + (ii * 32 + lm) * Band::STRIDE + (j * 32 + 8 * g + 4 * lh) * ES;
                    float v4[4];
#pragma unroll
                    for (int e = 0; e < 4; e++) v4[e] = sc((float)acc[i][j][4 * g + e], j, g, e);
                    if constexpr (OUT == 0)
                        *reinterpret_cast<float4 *>(dst) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                    else
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(cvt_pk_bf16(v4[0], v4[1]), cvt_pk_bf16(v4[2], v4[3]));
                }
            }
        }
        amax = fmaxf(amax, epi_band_to_global<ES, EPI>(band, y, M, N, m0 + wm * 128 + h * 64,
                                                        n0 + wn * 128, lane, vec));
    }
    if constexpr (AMAX) epi_tile_amax(amax, wave, lane, slot);
}

// fp32 accumulators -> y = (acc * gA) * gW (fp32 or bf16).  slot: the tile's
// entry of the fused-amax maxima (used with kEpiAmax only).
template <int OUT, int EPI = 0>
__device__ __forceinline__ void f32_band_epilogue(v16f (&acc)[4][4], uint8_t *lds, float gA,
                                                  float gW, int64_t M, int64_t N, int64_t m0,
                                                  int64_t n0, int wave, int wm, int wn, int lane,
                                                  void *y, float *slot = nullptr) {
    EpiScaleF32 sc{gA, gW};
    band_epilogue<OUT, EPI>(acc, sc, lds, M, N, m0, n0, wave, wm, wn, lane, y, slot);
}

// The epilogue of one 32-row slice i of a 128 x 128 quadrant of a split
// tile, run by a one-wave workgroup straight from the tile's partials (no
// accumulator array: a register-resident tile plus the loads in flight would
// spill).  A tail of T tiles so gets 16 T waves, enough to keep the partial
// reads in flight on every CU.  For each MFMA block (i, j), the lane's four
// 16-byte pieces of all S splits are loaded together, added in split order
// as T (int32: exact; fp32: fixed order), scaled by sc and written to a
// 32-row band, which then goes out as in band_epilogue.  part: the tile's
// first split; wave: the quadrant (the wave of the whole-tile kernels whose
// lanes' layout the partials follow).  The fused amax goes to *slot by an
// atomic max (the split kernel zeroed it; the maximum does not depend on the
// order).
constexpr int kFixupRows = 32;

template <int OUT, int EPI, class T, int S, class Scale>
__device__ __forceinline__ void split_fixup_epilogue(const uint32_t *part, Scale &sc, uint8_t *lds,
                                                     int64_t M, int64_t N, int64_t m0, int64_t n0,
                                                     int wave, int i, int lane, void *y, float *slot) {
    constexpr int ES = OUT == 1 ? 2 : 4;
    using Band = EpiBand<ES>;
    constexpr size_t kPieces = kSplitWords / 4;
    const uint4 *p4 = reinterpret_cast<const uint4 *>(part);
    const int wm = wave >> 1, wn = wave & 1, tid = wave * 64 + lane;
    const int lm = lane & 31, lh = lane >> 5;
    uint8_t *band = lds;
    const bool vec = ((N * ES) & 15) == 0;
    sc.row(m0 + wm * 128 + i * 32 + lm);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        uint4 v[S][4];
#pragma unroll
        for (int s = 0; s < S; s++)
#pragma unroll
            for (int g = 0; g < 4; g++) v[s][g] = p4[s * kPieces + ((i * 4 + j) * 4 + g) * 256 + tid];
#pragma unroll
        for (int g = 0; g < 4; g++) {
            T x[4] = {__builtin_bit_cast(T, v[0][g].x), __builtin_bit_cast(T, v[0][g].y),
                      __builtin_bit_cast(T, v[0][g].z), __builtin_bit_cast(T, v[0][g].w)};
#pragma unroll
            for (int s = 1; s < S; s++) {
                x[0] += __builtin_bit_cast(T, v[s][g].x);
                x[1] += __builtin_bit_cast(T, v[s][g].y);
                x[2] += __builtin_bit_cast(T, v[s][g].z);
                x[3] += __builtin_bit_cast(T, v[s][g].w);
            }
            float v4[4];
#pragma unroll
            for (int e = 0; e < 4; e++) v4[e] = sc((float)x[e], j, g, e);
            uint8_t *dst = band + lm * Band::STRIDE + (j * 32 + 8 * g + 4 * lh) * ES;
            if constexpr (OUT == 0)
                *reinterpret_cast<float4 *>(dst) = make_float4(v4[0], v4[1], v4[2], v4[3]);
            else
                *reinterpret_cast<uint2 *>(dst) = make_uint2(cvt_pk_bf16(v4[0], v4[1]), cvt_pk_bf16(v4[2], v4[3]));
        }
        // bound the loads in flight (one block's, two for few splits)
        if (S > 4 || (j & 1)) __builtin_amdgcn_sched_barrier(0);
    }
    float amax = epi_band_to_global<ES, EPI, kFixupRows>(band, y, M, N, m0 + wm * 128 + i * 32,
                                                         n0 + wn * 128, lane, vec);
    if constexpr ((EPI & kEpiAmax) != 0) {
        // non-negative floats order as their bit patterns
        amax = wave_max(amax);
        if (lane == 0) atomicMax(reinterpret_cast<unsigned *>(slot), __float_as_uint(amax));
    }
}

}  // namespace dmpq
