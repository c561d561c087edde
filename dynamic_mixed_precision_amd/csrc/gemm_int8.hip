// gemm_int8.hip -- INT8 quantized linear Y = (A W^T) * sA[m] * sW[n] on
// gfx950 i8 MFMA.  Method: 6Bit-Diffusion routes volatile layers to INT8
// activations against INT8-converted weights (gist.science summaries §2.A).
//
// Both operands are K-contiguous, the natural MFMA layout: one lane's
// 16-byte LDS read is a 16-value k-slice of one A row (or W row).  The k
// order inside an MFMA does not matter for the result: A and W fragments use
// the same k mapping and int32 addition is exact.  The W fragment is the
// MFMA's first operand, so the accumulators come out transposed and each lane
// stores 4 consecutive output columns at once.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid.  Workgroup tile 256 x 256,
// wave tile 128 x 128 = 4 x 4 MFMA 32x32x32 tiles (256 int32 accumulators per
// lane).  K advances 128 bytes per stage through a double-buffered LDS (rows
// padded to 144 bytes, conflict-free for the 32-row fragment reads); the
// next stage's global loads are in flight during the current stage's MFMAs,
// with one barrier per stage.
#include "device.hpp"
#include "gemm_common.hpp"
#include "gemm_dma.hpp"
#include "internal.hpp"

namespace dmpq {

namespace i8gemm {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int ROW = BK + 16;                  // padded LDS row, bytes
constexpr int STAGE = (BM + BN) * ROW;        // bytes per LDS stage
static_assert(4 * EpiBand<4>::BYTES <= 2 * STAGE, "epilogue bands fit in the stage buffers");
constexpr int LOADS = BM * BK / 16 / 256;     // 16-byte chunks per thread per operand
constexpr unsigned GROUP_M = 8;
}  // namespace i8gemm

// The tile's row and column scales, staged in LDS past the stage buffers:
// sA of rows m0 .. m0+255, then sW of columns n0 .. n0+255 (rows and columns
// past M or N load the last one; those outputs are never stored).  Each wave
// moves 64 of each with one LDS DMA (global_load_lds_dword) before its main
// loop issues the first stage, so the values need no registers and no wait
// of their own: the first stage's wait and barrier cover them, and the
// epilogue reads them from LDS instead of issuing 68 guarded global loads per
// lane after the last MFMA.
constexpr int kI8ScaleBytes = 512 * sizeof(float);
static_assert(2 * i8gemm::STAGE + kI8ScaleBytes <= 160 * 1024, "LDS of gemm_i8_kernel");
static_assert(gdma::LDS_BYTES + kI8ScaleBytes <= 160 * 1024, "LDS of gemm_i8_dma_kernel");
static_assert(gdma::LDS_BYTES % 16 == 0 && (2 * i8gemm::STAGE) % 16 == 0, "16-byte scale reads");

__device__ __forceinline__ void i8_scale_dma(float *scl, const float *sa, const float *sw, int64_t M,
                                             int64_t N, int64_t m0, int64_t n0, int tid) {
    typedef __attribute__((address_space(3))) void lds_void;
    const int wave = tid >> 6;
    const int64_t r = m0 + tid, c = n0 + tid;
    __builtin_amdgcn_global_load_lds((const void *)(sa + (r < M ? r : M - 1)),
                                     (lds_void *)(scl + 64 * wave), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((const void *)(sw + (c < N ? c : N - 1)),
                                     (lds_void *)(scl + 256 + 64 * wave), 4, 0, 0);
}

// Epilogue of both INT8 kernels, expanded in the kernel body (kept out of a
// function: as a function the compiler spills a few registers of it to
// scratch).  The MFMA runs with the W fragment as its first operand, so
// acc[i][j] holds the transposed block: lane l owns activation row m = l % 32
// of A-subtile i and, for register group g = r / 4, the four consecutive
// output columns 8g + 4*(l/32) + 0..3 of W-subtile j.  OUT 0/1: y =
// (float(acc) * sA[row]) * sW[col] (bit-exact in fp32), staged per wave
// through LDS in two 64-row bands and stored row-contiguous, with GELU and
// the fused amax per EPI; OUT 2: the raw int32 accumulators (test mode).  The
// stage buffers must be free (both main loops end with a barrier).  SCL: the
// tile's staged scales (i8_scale_dma).  pid: the tile's slot among the
// fused-amax maxima.
#define DMPQ_I8_EPILOGUE(SCL)                                                                     \
    {                                                                                             \
        constexpr int ES = OUT == 1 ? 2 : 4;                                                      \
        using Band = EpiBand<ES>;                                                                 \
        const int lm = lane & 31, lh = lane >> 5;                                                 \
        const float *scl_ = (SCL);                                                                \
        float4 swv[4][4];                                                                         \
        if constexpr (OUT != 2) {                                                                 \
            _Pragma("unroll") for (int j = 0; j < 4; j++)                                         \
                _Pragma("unroll") for (int g = 0; g < 4; g++) swv[j][g] =                         \
                    *reinterpret_cast<const float4 *>(scl_ + 256 + wn * 128 + j * 32 + 8 * g + 4 * lh); \
        }                                                                                         \
        uint8_t *band = reinterpret_cast<uint8_t *>(lds) + wave * Band::BYTES;                    \
        const bool vec = ((N * ES) & 15) == 0;                                                    \
        float amax = 0.0f;                                                                        \
        _Pragma("unroll") for (int h = 0; h < 2; h++) {                                           \
            _Pragma("unroll") for (int ii = 0; ii < 2; ii++) {                                    \
                const int i = 2 * h + ii;                                                         \
                const float sar = OUT == 2 ? 0.0f : scl_[wm * 128 + i * 32 + lm];                 \
                _Pragma("unroll") for (int j = 0; j < 4; j++) {                                   \
                    _Pragma("unroll") for (int g = 0; g < 4; g++) {                               \
                        uint8_t *dst = band + (ii * 32 + lm) * Band::STRIDE + (j * 32 + 8 * g + 4 * lh) * ES; \
                        if constexpr (OUT == 2) {                                                 \
                            *reinterpret_cast<int4 *>(dst) =                                      \
                                make_int4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], \
                                          acc[i][j][4 * g + 3]);                                  \
                        } else {                                                                  \
                            float v4[4];                                                          \
                            v4[0] = ((float)acc[i][j][4 * g + 0] * sar) * swv[j][g].x;            \
                            v4[1] = ((float)acc[i][j][4 * g + 1] * sar) * swv[j][g].y;            \
                            v4[2] = ((float)acc[i][j][4 * g + 2] * sar) * swv[j][g].z;            \
                            v4[3] = ((float)acc[i][j][4 * g + 3] * sar) * swv[j][g].w;            \
                            if constexpr (OUT == 0)                                               \
                                *reinterpret_cast<float4 *>(dst) = make_float4(v4[0], v4[1], v4[2], v4[3]); \
                            else                                                                  \
                                *reinterpret_cast<uint2 *>(dst) =                                 \
                                    make_uint2(cvt_pk_bf16(v4[0], v4[1]), cvt_pk_bf16(v4[2], v4[3])); \
                        }                                                                         \
                    }                                                                             \
                }                                                                                 \
            }                                                                                     \
            const float m = epi_band_to_global<ES, EPI>(band, y, M, N, m0 + wm * 128 + h * 64,    \
                                                        n0 + wn * 128, lane, vec);                \
            if constexpr ((EPI & kEpiAmax) != 0) amax = fmaxf(amax, m);                           \
        }                                                                                         \
        if constexpr ((EPI & kEpiAmax) != 0) epi_tile_amax(amax, wave, lane, partial + pid);      \
    }

template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ W,
    const float *__restrict__ sw, int64_t M, int64_t N, int64_t K, void *__restrict__ y,
    unsigned tiles_m, unsigned tiles_n, float *__restrict__ partial) {
    using namespace i8gemm;
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    // global -> register staging: chunk c = tid + 256*j covers row c/8, bytes
    // (c%8)*16.  Out-of-range chunks (ragged M, N or K) load from a clamped
    // in-range address; bit j of oka/okw records whether chunk j is real, and
    // the zeroing is applied only when the chunk is written to LDS, so the
    // loads stay in flight across the MFMAs.
    uint4 ra[LOADS], rw[LOADS];
    uint32_t oka = 0u, okw = 0u;
    const int nk = (int)((K + BK - 1) / BK);

#define DMPQ_I8_GLOAD(k0)                                                                    \
    oka = 0u;                                                                                \
    okw = 0u;                                                                                \
    _Pragma("unroll") for (int j = 0; j < LOADS; j++) {                                      \
        const int c = tid + 256 * j;                                                         \
        const int r = c >> 3;                                                                \
        const int64_t gk = (k0) + (c & 7) * 16;                                              \
        const int64_t gm = m0 + r, gn = n0 + r;                                              \
        const int64_t gkc = gk < K ? gk : K - 16;                                            \
        ra[j] = *reinterpret_cast<const uint4 *>(A + (gm < M ? gm : M - 1) * K + gkc);      \
        rw[j] = *reinterpret_cast<const uint4 *>(W + (gn < N ? gn : N - 1) * K + gkc);      \
        oka |= (uint32_t)(gm < M && gk < K) << j;                                            \
        okw |= (uint32_t)(gn < N && gk < K) << j;                                            \
    }
#define DMPQ_I8_SSTORE(buf)                                                                  \
    _Pragma("unroll") for (int j = 0; j < LOADS; j++) {                                      \
        const int c = tid + 256 * j;                                                         \
        const int r = c >> 3, kc = (c & 7) * 16;                                             \
        int8_t *base = lds + (buf) * STAGE;                                                  \
        const bool ia = (oka >> j) & 1u, iw = (okw >> j) & 1u;                               \
        *reinterpret_cast<uint4 *>(base + r * ROW + kc) =                                    \
            make_uint4(ia ? ra[j].x : 0u, ia ? ra[j].y : 0u, ia ? ra[j].z : 0u, ia ? ra[j].w : 0u); \
        *reinterpret_cast<uint4 *>(base + (BM + r) * ROW + kc) =                             \
            make_uint4(iw ? rw[j].x : 0u, iw ? rw[j].y : 0u, iw ? rw[j].z : 0u, iw ? rw[j].w : 0u); \
    }

    float *scl = reinterpret_cast<float *>(lds + 2 * STAGE);
    i8_scale_dma(scl, sa, sw, M, N, m0, n0, tid);
    DMPQ_I8_GLOAD(0)
    DMPQ_I8_SSTORE(0)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the scale DMA has landed
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            DMPQ_I8_GLOAD((int64_t)(kt + 1) * BK)
        }
        const int8_t *As = lds + cur * STAGE + (wm * 128 + (lane & 31)) * ROW + (lane >> 5) * 16;
        const int8_t *Ws = lds + cur * STAGE + (BM + wn * 128 + (lane & 31)) * ROW + (lane >> 5) * 16;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            v4i a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = *reinterpret_cast<const v4i *>(As + i * 32 * ROW + ks);
                b[i] = *reinterpret_cast<const v4i *>(Ws + i * 32 * ROW + ks);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j], a[i], acc[i][j], 0, 0, 0);
        }
        if (more) {
            DMPQ_I8_SSTORE(cur ^ 1)
        }
        __syncthreads();
    }
#undef DMPQ_I8_GLOAD
#undef DMPQ_I8_SSTORE

    DMPQ_I8_EPILOGUE(scl)
}

// ---------------------------------------------------------------------------
// INT8 GEMM against an NVFP4 weight converted in the weight-tile load
// (gist.science Chinese summary §2.A: weights are kept in NVFP4 and converted
// when an INT8 GEMM needs them).  The weight tile of each stage is loaded as
// NVFP4 codes and E4M3 scales (0.5625 bytes per element instead of 1) and
// requantized to INT8 in registers with the per-row reciprocal of
// w8_row_scales_kernel, by the same operations in the same order as the
// separate conversion (nvfp4_block_values, then int8_codes_magic), before it
// is written to LDS; a row with s_row 0 codes as zeros.  The B operand is
// therefore the separately converted weight bit for bit, and so is the
// result.  The main loop is the register-staged one of gemm_i8_kernel
// (K % 128 == 0 here, rows past M or N load a clamped row whose outputs are
// never stored, so no masks): the loads of stage kt+1 are in flight during
// stage kt's MFMAs, and the conversion runs when they are written to LDS.
// Weight staging: piece p = tid + 256 j (j < 4) is 32 elements of row p / 4 =
// tid / 4 + 64 j, the 16 code bytes and 2 scale bytes at piece p % 4 of the
// stage, so a thread's four rows are fixed for the whole K loop.
// ---------------------------------------------------------------------------
template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_i8w4_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const uint8_t *__restrict__ cw,
    const uint8_t *__restrict__ sw, const float *__restrict__ gw, const float *__restrict__ s_row,
    const float *__restrict__ inv_row, int64_t M, int64_t N, int64_t K, void *__restrict__ y,
    unsigned tiles_m, unsigned tiles_n, float *__restrict__ partial) {
    using namespace i8gemm;
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    constexpr int WP = 4;  // weight pieces per thread per stage
    const int piece = tid & 3;
    const uint8_t *wc[WP];
    const uint16_t *ws2[WP];
    float inv[WP];
    bool zrow[WP];
    const float g = *gw;
#pragma unroll
    for (int j = 0; j < WP; j++) {
        const int64_t r = n0 + (tid >> 2) + 64 * j;
        const int64_t gn = r < N ? r : N - 1;
        wc[j] = cw + gn * (K / 2) + piece * 16;
        ws2[j] = reinterpret_cast<const uint16_t *>(sw + gn * (K / 16) + piece * 2);
        inv[j] = inv_row[gn];
        zrow[j] = s_row[gn] == 0.0f;
    }
    uint4 ra[LOADS], rc[WP];
    uint32_t rs[WP];
    const int nk = (int)(K / BK);

#define DMPQ_I8W4_GLOAD(k0)                                                                  \
    _Pragma("unroll") for (int j = 0; j < LOADS; j++) {                                      \
        const int c = tid + 256 * j;                                                         \
        const int64_t gm = m0 + (c >> 3);                                                    \
        ra[j] = *reinterpret_cast<const uint4 *>(A + (gm < M ? gm : M - 1) * K + (k0) + (c & 7) * 16); \
    }                                                                                        \
    _Pragma("unroll") for (int j = 0; j < WP; j++) {                                         \
        rc[j] = *reinterpret_cast<const uint4 *>(wc[j] + (k0) / 2);                           \
        rs[j] = ws2[j][(k0) / 32];                                                           \
    }
#define DMPQ_I8W4_SSTORE(buf)                                                                \
    {                                                                                        \
        int8_t *base = lds + (buf) * STAGE;                                                  \
        _Pragma("unroll") for (int j = 0; j < LOADS; j++) {                                  \
            const int c = tid + 256 * j;                                                     \
            *reinterpret_cast<uint4 *>(base + (c >> 3) * ROW + (c & 7) * 16) = ra[j];         \
        }                                                                                    \
        _Pragma("unroll") for (int j = 0; j < WP; j++) {                                     \
            float v[16];                                                                     \
            uint4 q0 = make_uint4(0u, 0u, 0u, 0u), q1 = q0;                                  \
            nvfp4_block_values(make_uint2(rc[j].x, rc[j].y), e4m3_value(rs[j] & 0xFFu), g, v); \
            if (!zrow[j]) q0 = int8_codes_magic(v, inv[j]);                                  \
            nvfp4_block_values(make_uint2(rc[j].z, rc[j].w), e4m3_value(rs[j] >> 8), g, v);  \
            if (!zrow[j]) q1 = int8_codes_magic(v, inv[j]);                                  \
            int8_t *dst = base + (BM + (tid >> 2) + 64 * j) * ROW + piece * 32;              \
            *reinterpret_cast<uint4 *>(dst) = q0;                                            \
            *reinterpret_cast<uint4 *>(dst + 16) = q1;                                       \
        }                                                                                    \
    }

    float *scl = reinterpret_cast<float *>(lds + 2 * STAGE);
    i8_scale_dma(scl, sa, s_row, M, N, m0, n0, tid);
    DMPQ_I8W4_GLOAD((int64_t)0)
    DMPQ_I8W4_SSTORE(0)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the scale DMA has landed
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        // unconditional (the last stage reloads itself, in bounds): under a
        // branch the compiler keeps the staged A chunks in scratch memory
        DMPQ_I8W4_GLOAD((int64_t)(more ? kt + 1 : kt) * BK)
        const int8_t *As = lds + cur * STAGE + (wm * 128 + (lane & 31)) * ROW + (lane >> 5) * 16;
        const int8_t *Ws = lds + cur * STAGE + (BM + wn * 128 + (lane & 31)) * ROW + (lane >> 5) * 16;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            v4i a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = *reinterpret_cast<const v4i *>(As + i * 32 * ROW + ks);
                b[i] = *reinterpret_cast<const v4i *>(Ws + i * 32 * ROW + ks);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j], a[i], acc[i][j], 0, 0, 0);
        }
        if (more) {
            DMPQ_I8W4_SSTORE(cur ^ 1)
        }
        __syncthreads();
    }
#undef DMPQ_I8W4_GLOAD
#undef DMPQ_I8W4_SSTORE

    DMPQ_I8_EPILOGUE(scl)
}

// ---------------------------------------------------------------------------
// Fast path for K % 128 == 0: the DMA-fed main loop of gemm_dma.hpp with i8
// MFMA (v_mfma_i32_32x32x32_i8), then the scaled epilogue.
// ---------------------------------------------------------------------------
template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_i8_dma_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ W,
    const float *__restrict__ sw, int64_t M, int64_t N, int64_t K, void *__restrict__ y,
    unsigned tiles_m, unsigned tiles_n, float *__restrict__ partial) {
    using namespace gdma;
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;

    float *scl = reinterpret_cast<float *>(lds + LDS_BYTES);
    i8_scale_dma(scl, sa, sw, M, N, m0, n0, tid);  // older than the first stage's DMA
    v16i acc[4][4];
    dma_gemm_mainloop<OpI8, false>(reinterpret_cast<const uint8_t *>(A),
                                   reinterpret_cast<const uint8_t *>(W), M, N, K, K, m0, n0,
                                   reinterpret_cast<uint8_t *>(lds), acc);
    DMPQ_I8_EPILOGUE(scl)
}

// The split workgroups of a SplitPlan launch: the main loop over this
// workgroup's K stages, then the raw int32 accumulators to the split area.
// The first split of a tile also zeroes the tile's fused-amax slot (partial
// may be NULL), which the fixup then raises by atomic max.
__global__ __launch_bounds__(256, 1) void gemm_i8_split_kernel(
    const int8_t *__restrict__ A, const int8_t *__restrict__ W, int64_t M, int64_t N, int64_t K,
    unsigned tiles_m, unsigned tiles_n, SplitPlan sp, uint32_t *__restrict__ spart,
    float *__restrict__ partial) {
    using namespace gdma;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    const SplitUnit u = split_unit(sp, tiles_m, tiles_n, GROUP_M);
    if (partial && u.kt0 == 0 && threadIdx.x == 0) partial[sp.full + blockIdx.x / sp.splits] = 0.0f;
    const int64_t k0 = (int64_t)u.kt0 * BK;
    v16i acc[4][4];
    dma_gemm_mainloop<OpI8, false>(reinterpret_cast<const uint8_t *>(A) + k0,
                                   reinterpret_cast<const uint8_t *>(W) + k0, M, N, K,
                                   (int64_t)u.kt1 * BK - k0, (int64_t)u.tc.m * BM, (int64_t)u.tc.n * BN,
                                   lds8, acc);
    store_split_partial(acc, spart + (size_t)blockIdx.x * kSplitWords, threadIdx.x);
}

// Output scaling of the INT8 fixup: y = (float(acc) * sA[row]) * sW[col],
// bit-exact in fp32.
struct EpiScaleI8 {
    const float *sa;
    int64_t M;
    float sar;
    float swv[4][4][4];  // the lane's 64 column scales, 0 past N
    // c0: first output column of the lane's (j, g) groups.  The loads are
    // clamped and unconditional, so they issue back to back without branches.
    __device__ __forceinline__ EpiScaleI8(const float *sa_, const float *sw, int64_t M_, int64_t N,
                                          int64_t c0)
        : sa(sa_), M(M_), sar(0.0f) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int g = 0; g < 4; g++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int64_t col = c0 + j * 32 + 8 * g + e;
                    const float v = sw[col < N ? col : N - 1];
                    swv[j][g][e] = col < N ? v : 0.0f;
                }
    }
    __device__ __forceinline__ void row(int64_t r) {
        const float v = sa[r < M ? r : M - 1];
        sar = r < M ? v : 0.0f;
    }
    __device__ __forceinline__ float operator()(float a, int j, int g, int e) const {
        return (a * sar) * swv[j][g][e];
    }
};

// The tail tiles of a split launch: the int32 partials of each tile's split
// workgroups added in split order (exact), then the same scaled epilogue.
// One workgroup of one wave per 32-row slice of a 128 x 128 quadrant (16 per
// tail tile).
template <int OUT, int EPI, int S>
__global__ __launch_bounds__(64) void gemm_i8_fixup_kernel(
    const float *__restrict__ sa, const float *__restrict__ sw, int64_t M, int64_t N,
    void *__restrict__ y, unsigned tiles_m, unsigned tiles_n, float *__restrict__ partial,
    SplitPlan sp, const uint32_t *__restrict__ spart) {
    using namespace gdma;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds8[];
    // workgroup = (tail tile t, quadrant wave, 32-row slice i)
    const int lane = threadIdx.x, i = blockIdx.x & 3, wave = (blockIdx.x >> 2) & 3;
    const unsigned t = blockIdx.x >> 4, pid = sp.full + t;
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;
    EpiScaleI8 sc(sa, sw, M, N, n0 + (wave & 1) * 128 + 4 * (lane >> 5));
    split_fixup_epilogue<OUT, EPI, int, S>(spart + (size_t)t * S * kSplitWords, sc, lds8, M, N, m0, n0, wave,
                                           i, lane, y, (EPI & kEpiAmax) ? partial + pid : nullptr);
}

template <class KernelFn>
static hipError_t allow_lds(KernelFn fn, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// spart: the split area (kSplitAreaBytes), or NULL for no split.
template <int OUT, int EPI>
static hipError_t launch_i8_paths(hipStream_t s, const int8_t *qa, const float *sa, const int8_t *qw,
                                  const float *sw, int64_t M, int64_t N, int64_t K, void *y,
                                  float *partial, uint32_t *spart) {
    constexpr bool CAN_SPLIT = OUT != 2;
    // Kernels need more dynamic LDS than the default limit: opt in once.
    static const hipError_t attr = [] {
        hipError_t e = allow_lds(gemm_i8_kernel<OUT, EPI>, 2 * i8gemm::STAGE + kI8ScaleBytes);
        if (e == hipSuccess) e = allow_lds(gemm_i8_dma_kernel<OUT, EPI>, gdma::LDS_BYTES + kI8ScaleBytes);
        if (e == hipSuccess) e = allow_lds(gemm_i8_split_kernel, gdma::LDS_BYTES);

        return e;
    }();
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
    const dim3 block(256);
    const unsigned utm = (unsigned)tm, utn = (unsigned)tn;
    if (K % gdma::BK != 0) {
        hipLaunchKernelGGL((gemm_i8_kernel<OUT, EPI>), dim3((unsigned)(tm * tn)), block,
                           2 * i8gemm::STAGE + kI8ScaleBytes, s, qa,
                           sa, qw, sw, M, N, K, y, utm, utn, partial);
        return hipGetLastError();
    }
    const SplitPlan sp = plan_split(tm * tn, (int)(K / gdma::BK), CAN_SPLIT && spart != nullptr && K >= kSplitMinKInt8);
    if (sp.full > 0) {
        hipLaunchKernelGGL((gemm_i8_dma_kernel<OUT, EPI>), dim3(sp.full), block,
                           gdma::LDS_BYTES + kI8ScaleBytes, s, qa, sa, qw,
                           sw, M, N, K, y, utm, utn, partial);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if constexpr (CAN_SPLIT) {
        if (sp.splits > 1) {
            hipLaunchKernelGGL(gemm_i8_split_kernel, dim3(sp.tail * sp.splits), block, gdma::LDS_BYTES, s, qa, qw,
                               M, N, K, utm, utn, sp, spart, (EPI & kEpiAmax) ? partial : nullptr);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const dim3 fg(16 * sp.tail), fb(64);
            const size_t fl = (size_t)kFixupRows * EpiBand<OUT == 1 ? 2 : 4>::STRIDE;
            const uint32_t *cp = spart;
#define DMPQ_I8_FIX(S_)                                                                          \
    case S_:                                                                                     \
        hipLaunchKernelGGL((gemm_i8_fixup_kernel<OUT, EPI, S_>), fg, fb, fl, s, sa, sw, M, N, y, utm, utn, \
                           partial, sp, cp);                                                     \
        break;
            switch (sp.splits) {
                DMPQ_I8_FIX(2) DMPQ_I8_FIX(3) DMPQ_I8_FIX(4) DMPQ_I8_FIX(8)
                default: return hipErrorInvalidValue;
            }
#undef DMPQ_I8_FIX
        }
    }
    return hipGetLastError();
}

template <int OUT, int EPI>
static hipError_t launch_i8w4(hipStream_t s, const int8_t *qa, const float *sa, const uint8_t *cw,
                              const uint8_t *sw, const float *gw, const float *s_row, const float *inv_row,
                              int64_t M, int64_t N, int64_t K, void *y, float *partial) {
    static const hipError_t attr = allow_lds(gemm_i8w4_kernel<OUT, EPI>, 2 * i8gemm::STAGE + kI8ScaleBytes);
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
    hipLaunchKernelGGL((gemm_i8w4_kernel<OUT, EPI>), dim3((unsigned)(tm * tn)), dim3(256),
                       2 * i8gemm::STAGE + kI8ScaleBytes, s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y,
                       (unsigned)tm, (unsigned)tn, partial);
    return hipGetLastError();
}

hipError_t launch_gemm_int8_w4(hipStream_t s, const int8_t *qa, const float *sa, const uint8_t *cw,
                               const uint8_t *sw, const float *gw, const float *s_row,
                               const float *inv_row, int64_t M, int64_t N, int64_t K, int out_dtype,
                               void *y, int epi, float *partial) {
    if (M == 0 || N == 0) return hipSuccess;
    if (K % i8gemm::BK != 0) return hipErrorInvalidValue;
    if (epi == 0) {
        switch (out_dtype) {
            case 0: return launch_i8w4<0, 0>(s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y, partial);
            case 1: return launch_i8w4<1, 0>(s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y, partial);
            case 2: return launch_i8w4<2, 0>(s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y, partial);
        }
        return hipErrorInvalidValue;
    }
    if (out_dtype != 1) return hipErrorInvalidValue;
    switch (epi) {
        case 1: return launch_i8w4<1, 1>(s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y, partial);
        case 2: return launch_i8w4<1, 2>(s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y, partial);
        case 3: return launch_i8w4<1, 3>(s, qa, sa, cw, sw, gw, s_row, inv_row, M, N, K, y, partial);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_int8(hipStream_t s, const int8_t *qa, const float *sa, const int8_t *qw,
                            const float *sw, int64_t M, int64_t N, int64_t K, int out_dtype,
                            void *y, int epi, float *partial, uint32_t *spart) {
    if (M == 0 || N == 0) return hipSuccess;
    if (epi == 0) {
        switch (out_dtype) {
            case 0: return launch_i8_paths<0, 0>(s, qa, sa, qw, sw, M, N, K, y, partial, spart);
            case 1: return launch_i8_paths<1, 0>(s, qa, sa, qw, sw, M, N, K, y, partial, spart);
            case 2: return launch_i8_paths<2, 0>(s, qa, sa, qw, sw, M, N, K, y, partial, spart);
        }
        return hipErrorInvalidValue;
    }
    if (out_dtype != 1) return hipErrorInvalidValue;
    switch (epi) {
        case 1: return launch_i8_paths<1, 1>(s, qa, sa, qw, sw, M, N, K, y, partial, spart);
        case 2: return launch_i8_paths<1, 2>(s, qa, sa, qw, sw, M, N, K, y, partial, spart);
        case 3: return launch_i8_paths<1, 3>(s, qa, sa, qw, sw, M, N, K, y, partial, spart);
    }
    return hipErrorInvalidValue;
}

}  // namespace dmpq
