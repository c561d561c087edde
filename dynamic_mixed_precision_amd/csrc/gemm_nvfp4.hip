// gemm_nvfp4.hip -- NVFP4 quantized linear on gfx950.  Method: 6Bit-Diffusion
// routes temporally stable layers to NVFP4 (E2M1 elements, one E4M3 scale
// per 16, an fp32 tensor scale) against NVFP4 weights (gist.science
// summaries §1 and §2.A).
//
// gfx950's block-scaled MFMA applies one power-of-two (E8M0) scale per 32
// elements, which cannot carry an E4M3 scale per 16 exactly.  This kernel
// dequantizes exactly instead: an E2M1 value (<= 2 significant bits) times an
// E4M3 scale (<= 4 significant bits) has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in fp16 (11 bits, normal from 2^-14).  The
// fp16 MFMA products are exact in fp32; only the fp32 accumulation rounds.
// Epilogue y = (acc * gA) * gW.
//
// Dequant per code byte: v_cvt_scalef32_pk_f16_fp4 (scale 1.0; that
// converter uses only the exponent of its scale operand, so the E4M3 scale is
// applied separately) gives two fp16 values, then one v_pk_mul_f16 by the
// block's scale.
//
// Tiling (all paths of variant 0): 256 threads = 2 x 2 waves, workgroup tile
// 256 x 256, wave tile 128 x 128 = 4 x 4 MFMA 32x32x16 tiles.  Three paths:
//  * K % 128 == 0 (the DiT shapes; K >= 384 when K % 256 != 0): raw codes
//    and scales are copied into LDS by DMA and each wave dequantizes its own
//    fragments into registers (gemm_fp4_dma_kernel; gemm_fp4_dma_tail_kernel
//    when K % 256 == 128, whose last stage is a half stage);
//  * K % 64 == 0: codes are loaded into registers, dequantized once per
//    workgroup into a double-buffered fp16 LDS tile (gemm_fp4_fast_kernel);
//  * any K % 16 == 0: as the previous, with the K tail masked
//    (gemm_fp4_f16_kernel).
// Variant 1 (gemm_fp4_scaled_kernel) uses the block-scaled MFMA instead.
#include "device.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace dmpq {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));

namespace fp4gemm {
constexpr int BM = 256, BN = 256, BKE = 64;  // BKE: k elements per stage
constexpr int ROW = BKE * 2 + 16;            // padded LDS row, bytes (fp16)
constexpr int STAGE = (BM + BN) * ROW;
static_assert(4 * EpiBand<4>::BYTES <= 2 * STAGE, "epilogue bands fit in the stage buffers");
constexpr unsigned GROUP_M = 8;
}  // namespace fp4gemm

// 32 codes (16 bytes, two 16-element scale groups) -> 32 fp16, as 16 words.
__device__ __forceinline__ void dequant32(const uint4 c, uint32_t s01, uint32_t out[16]) {
    const v2h s0 = (v2h){(_Float16)e4m3_value(s01 & 0xFFu), (_Float16)e4m3_value(s01 & 0xFFu)};
    const v2h s1 = (v2h){(_Float16)e4m3_value(s01 >> 8), (_Float16)e4m3_value(s01 >> 8)};
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const v2h sc = i < 2 ? s0 : s1;
        const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0) * sc;
        const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1) * sc;
        const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2) * sc;
        const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3) * sc;
        out[4 * i + 0] = __builtin_bit_cast(uint32_t, p0);
        out[4 * i + 1] = __builtin_bit_cast(uint32_t, p1);
        out[4 * i + 2] = __builtin_bit_cast(uint32_t, p2);
        out[4 * i + 3] = __builtin_bit_cast(uint32_t, p3);
    }
}

// As dequant32, with the two E4M3 scale codes in the low 16 bits of s01
// decoded by v_cvt_scalef32_pk_f16_fp8 (scale 1.0; every finite OCP E4M3
// value is exact in fp16).
__device__ __forceinline__ void dequant32_fast(const uint4 c, uint32_t s01, uint32_t out[16]) {
    const v2h s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s01, 1.0f, false);
    const v2h s0 = __builtin_shufflevector(s, s, 0, 0);
    const v2h s1 = __builtin_shufflevector(s, s, 1, 1);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const v2h sc = i < 2 ? s0 : s1;
        out[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0) * sc);
        out[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1) * sc);
        out[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2) * sc);
        out[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3) * sc);
    }
}

// Epilogue of the NVFP4 kernels: y = (acc * gA) * gW through the per-wave LDS
// bands (callers end their main loop with a barrier, so the stage buffers are
// free); pid: the tile's slot among the fused-amax maxima.
template <int OUT, int EPI>
__device__ __forceinline__ void fp4_epilogue(v16f (&acc)[4][4], uint8_t *lds, const float *ga,
                                             const float *gw, int64_t M, int64_t N, int64_t m0,
                                             int64_t n0, int wave, int wm, int wn, int lane,
                                             void *y, float *partial, unsigned pid) {
    f32_band_epilogue<OUT, EPI>(acc, lds, *ga, *gw, M, N, m0, n0, wave, wm, wn, lane, y,
                                (EPI & kEpiAmax) ? partial + pid : nullptr);
}

template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_fp4_f16_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n,
    float *__restrict__ partial) {
    using namespace fp4gemm;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;
    const int64_t nb = K / 16;  // scale groups per row
    const int64_t rb = K / 2;   // code bytes per row

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    // Staging: chunk c = tid + 256*h (h = 0, 1) is row c/2, k-half c%2 of a
    // stage (16 code bytes = 32 elements = 2 scale groups).  Two register sets
    // (stage s lives in set s & 1) keep the global loads one full stage ahead.
    // Out-of-range groups read a clamped in-range address and a bit of `ok`
    // records whether they are real; zeroing happens at dequant time.
    uint2 rca0[2][2], rcw0[2][2], rca1[2][2], rcw1[2][2];
    uint32_t rsa0[2][2], rsw0[2][2], rsa1[2][2], rsw1[2][2];
    uint32_t ok0 = 0u, ok1 = 0u;  // bit 4h+q: A group q, bit 4h+2+q: W group q
    const int nk = (int)((nb + 3) / 4);

#define DMPQ_F4_GLOAD(SET, g0)                                                                \
    ok##SET = 0u;                                                                             \
    _Pragma("unroll") for (int h = 0; h < 2; h++) {                                           \
        const int c = tid + 256 * h;                                                          \
        const int r = c >> 1;                                                                 \
        const int64_t gm = m0 + r, gn = n0 + r;                                               \
        const int64_t gmc = gm < M ? gm : M - 1, gnc = gn < N ? gn : N - 1;                   \
        _Pragma("unroll") for (int q = 0; q < 2; q++) {                                       \
            const int64_t gi = (g0) + 2 * (c & 1) + q;                                        \
            const int64_t gic = gi < nb ? gi : nb - 1;                                        \
            rca##SET[h][q] = *reinterpret_cast<const uint2 *>(ca + gmc * rb + 8 * gic);       \
            rcw##SET[h][q] = *reinterpret_cast<const uint2 *>(cw + gnc * rb + 8 * gic);       \
            rsa##SET[h][q] = sa[gmc * nb + gic];                                              \
            rsw##SET[h][q] = sw[gnc * nb + gic];                                              \
            ok##SET |= (uint32_t)(gm < M && gi < nb) << (4 * h + q);                          \
            ok##SET |= (uint32_t)(gn < N && gi < nb) << (4 * h + 2 + q);                      \
        }                                                                                     \
    }
    // Dequantize one quarter of a staged stage (part p: A/W of chunk h = p/2)
    // into LDS buffer buf.
#define DMPQ_F4_DQ(SET, buf, p)                                                               \
    {                                                                                         \
        const int h = (p) >> 1, isw = (p) & 1;                                                \
        const int c = tid + 256 * h;                                                          \
        const int r = c >> 1;                                                                 \
        uint8_t *dst = lds + (buf) * STAGE + ((isw ? BM : 0) + r) * ROW + (c & 1) * 64;       \
        const uint2 *cc = isw ? rcw##SET[h] : rca##SET[h];                                    \
        const uint32_t *ss = isw ? rsw##SET[h] : rsa##SET[h];                                 \
        const bool k0 = (ok##SET >> (4 * h + 2 * isw)) & 1u;                                  \
        const bool k1 = (ok##SET >> (4 * h + 2 * isw + 1)) & 1u;                              \
        uint32_t d[16];                                                                       \
        dequant32(make_uint4(k0 ? cc[0].x : 0u, k0 ? cc[0].y : 0u, k1 ? cc[1].x : 0u,         \
                             k1 ? cc[1].y : 0u),                                              \
                  (k0 ? ss[0] : 0u) | ((k1 ? ss[1] : 0u) << 8), d);                           \
        _Pragma("unroll") for (int q = 0; q < 4; q++)                                         \
            *reinterpret_cast<uint4 *>(dst + 16 * q) =                                        \
                make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);               \
    }
    // Fragments of k-step s (16 k-elements = 32 bytes) of LDS buffer buf.
#define DMPQ_F4_FRAG(dsta, dstb, buf, s)                                                      \
    {                                                                                         \
        const uint8_t *As = lds + (buf) * STAGE + (wm * 128 + (lane & 31)) * ROW + (lane >> 5) * 16 + 32 * (s); \
        const uint8_t *Ws = lds + (buf) * STAGE + (BM + wn * 128 + (lane & 31)) * ROW + (lane >> 5) * 16 + 32 * (s); \
        _Pragma("unroll") for (int i = 0; i < 4; i++) {                                       \
            dsta[i] = *reinterpret_cast<const v8h *>(As + i * 32 * ROW);                      \
            dstb[i] = *reinterpret_cast<const v8h *>(Ws + i * 32 * ROW);                      \
        }                                                                                     \
    }
#define DMPQ_F4_MFMA(fa, fb)                                                                  \
    _Pragma("unroll") for (int i = 0; i < 4; i++)                                             \
        _Pragma("unroll") for (int j = 0; j < 4; j++)                                         \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    // One stage kt (parity P): first the global loads of stage kt+2 into
    // register set P (its stage kt was dequantized during stage kt-1), then the
    // MFMAs on LDS buffer P interleaved with the dequant of stage kt+1
    // (register set 1-P) into LDS buffer 1-P.
#define DMPQ_F4_ITER(P, Q)                                                                    \
    {                                                                                         \
        v8h fa0[4], fb0[4], fa1[4], fb1[4];                                                   \
        const bool more = kt + 1 < nk;                                                        \
        if (kt + 2 < nk) {                                                                    \
            DMPQ_F4_GLOAD(P, (int64_t)(kt + 2) * 4)                                           \
        }                                                                                     \
        DMPQ_F4_FRAG(fa0, fb0, P, 0)                                                          \
        DMPQ_F4_FRAG(fa1, fb1, P, 1)                                                          \
        DMPQ_F4_MFMA(fa0, fb0)                                                                \
        if (more) DMPQ_F4_DQ(Q, Q, 0)                                                         \
        DMPQ_F4_FRAG(fa0, fb0, P, 2)                                                          \
        DMPQ_F4_MFMA(fa1, fb1)                                                                \
        if (more) DMPQ_F4_DQ(Q, Q, 1)                                                         \
        DMPQ_F4_FRAG(fa1, fb1, P, 3)                                                          \
        DMPQ_F4_MFMA(fa0, fb0)                                                                \
        if (more) DMPQ_F4_DQ(Q, Q, 2)                                                         \
        DMPQ_F4_MFMA(fa1, fb1)                                                                \
        if (more) DMPQ_F4_DQ(Q, Q, 3)                                                         \
        __syncthreads();                                                                      \
    }

    DMPQ_F4_GLOAD(0, 0)
    if (nk > 1) {
        DMPQ_F4_GLOAD(1, 4)
    }
    DMPQ_F4_DQ(0, 0, 0)
    DMPQ_F4_DQ(0, 0, 1)
    DMPQ_F4_DQ(0, 0, 2)
    DMPQ_F4_DQ(0, 0, 3)
    __syncthreads();
    // Stage kt uses LDS buffer kt & 1; stage kt+1 is dequantized from register
    // set (kt+1) & 1; stage kt+2 is loaded into set kt & 1 (already consumed).
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        DMPQ_F4_ITER(0, 1)
        kt++;
        DMPQ_F4_ITER(1, 0)
        kt--;
    }
    if (kt < nk) DMPQ_F4_ITER(0, 1)
#undef DMPQ_F4_GLOAD
#undef DMPQ_F4_DQ
#undef DMPQ_F4_FRAG
#undef DMPQ_F4_MFMA
#undef DMPQ_F4_ITER

    fp4_epilogue<OUT, EPI>(acc, lds, ga, gw, M, N, m0, n0, wave, wm, wn, lane, y, partial, pid);
}

// ---------------------------------------------------------------------------
// Fast path for K % 64 == 0 (every stage is full): no K tail to zero, and
// rows past M or N only feed outputs that are never stored, so operands load
// from clamped rows without any masking.  Each staged chunk is one 16-byte
// code load and one 2-byte scale load from per-lane pointers fixed for the
// whole K loop; scales are decoded by the hardware fp8 converter.
// ---------------------------------------------------------------------------
template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_fp4_fast_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n,
    float *__restrict__ partial) {
    using namespace fp4gemm;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;
    const int64_t nb = K / 16, rb = K / 2;
    const int nk = (int)(nb / 4);

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    // chunk h (h = 0, 1) of this thread: row (tid + 256h) / 2, k-half tid % 2
    const uint8_t *pa[2], *pw[2], *qa[2], *qw[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const int c = tid + 256 * h, r = c >> 1;
        const int64_t gm = m0 + r < M ? m0 + r : M - 1;
        const int64_t gn = n0 + r < N ? n0 + r : N - 1;
        pa[h] = ca + gm * rb + 16 * (c & 1);
        pw[h] = cw + gn * rb + 16 * (c & 1);
        qa[h] = sa + gm * nb + 2 * (c & 1);
        qw[h] = sw + gn * nb + 2 * (c & 1);
    }
    uint4 xa0[2], xw0[2], xa1[2], xw1[2];
    uint32_t ya0[2], yw0[2], ya1[2], yw1[2];

#define DMPQ_F4F_GLOAD(SET, st)                                                                \
    _Pragma("unroll") for (int h = 0; h < 2; h++) {                                            \
        xa##SET[h] = *reinterpret_cast<const uint4 *>(pa[h] + 32 * (int64_t)(st));             \
        xw##SET[h] = *reinterpret_cast<const uint4 *>(pw[h] + 32 * (int64_t)(st));             \
        ya##SET[h] = *reinterpret_cast<const uint16_t *>(qa[h] + 4 * (int64_t)(st));           \
        yw##SET[h] = *reinterpret_cast<const uint16_t *>(qw[h] + 4 * (int64_t)(st));           \
    }
#define DMPQ_F4F_DQ(SET, buf, p)                                                               \
    {                                                                                          \
        const int h = (p) >> 1, isw = (p) & 1;                                                 \
        const int c = tid + 256 * h;                                                           \
        uint8_t *dst = lds + (buf) * STAGE + ((isw ? BM : 0) + (c >> 1)) * ROW + (c & 1) * 64; \
        uint32_t d[16];                                                                        \
        dequant32_fast(isw ? xw##SET[h] : xa##SET[h], isw ? yw##SET[h] : ya##SET[h], d);       \
        _Pragma("unroll") for (int q = 0; q < 4; q++)                                          \
            *reinterpret_cast<uint4 *>(dst + 16 * q) =                                         \
                make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]);                \
    }
#define DMPQ_F4F_FRAG(dsta, dstb, buf, s)                                                      \
    {                                                                                          \
        const uint8_t *As = lds + (buf) * STAGE + (wm * 128 + (lane & 31)) * ROW + (lane >> 5) * 16 + 32 * (s); \
        const uint8_t *Ws = lds + (buf) * STAGE + (BM + wn * 128 + (lane & 31)) * ROW + (lane >> 5) * 16 + 32 * (s); \
        _Pragma("unroll") for (int i = 0; i < 4; i++) {                                        \
            dsta[i] = *reinterpret_cast<const v8h *>(As + i * 32 * ROW);                       \
            dstb[i] = *reinterpret_cast<const v8h *>(Ws + i * 32 * ROW);                       \
        }                                                                                      \
    }
#define DMPQ_F4F_MFMA(fa, fb)                                                                  \
    _Pragma("unroll") for (int i = 0; i < 4; i++)                                              \
        _Pragma("unroll") for (int j = 0; j < 4; j++)                                          \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
#define DMPQ_F4F_ITER(P, Q)                                                                    \
    {                                                                                          \
        v8h fa0[4], fb0[4], fa1[4], fb1[4];                                                    \
        const bool more = kt + 1 < nk;                                                         \
        if (kt + 2 < nk) {                                                                     \
            DMPQ_F4F_GLOAD(P, kt + 2)                                                          \
        }                                                                                      \
        DMPQ_F4F_FRAG(fa0, fb0, P, 0)                                                          \
        DMPQ_F4F_FRAG(fa1, fb1, P, 1)                                                          \
        DMPQ_F4F_MFMA(fa0, fb0)                                                                \
        if (more) DMPQ_F4F_DQ(Q, Q, 0)                                                         \
        DMPQ_F4F_FRAG(fa0, fb0, P, 2)                                                          \
        DMPQ_F4F_MFMA(fa1, fb1)                                                                \
        if (more) DMPQ_F4F_DQ(Q, Q, 1)                                                         \
        DMPQ_F4F_FRAG(fa1, fb1, P, 3)                                                          \
        DMPQ_F4F_MFMA(fa0, fb0)                                                                \
        if (more) DMPQ_F4F_DQ(Q, Q, 2)                                                         \
        DMPQ_F4F_MFMA(fa1, fb1)                                                                \
        if (more) DMPQ_F4F_DQ(Q, Q, 3)                                                         \
        __syncthreads();                                                                       \
    }

    DMPQ_F4F_GLOAD(0, 0)
    if (nk > 1) {
        DMPQ_F4F_GLOAD(1, 1)
    }
    DMPQ_F4F_DQ(0, 0, 0)
    DMPQ_F4F_DQ(0, 0, 1)
    DMPQ_F4F_DQ(0, 0, 2)
    DMPQ_F4F_DQ(0, 0, 3)
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        DMPQ_F4F_ITER(0, 1)
        kt++;
        DMPQ_F4F_ITER(1, 0)
        kt--;
    }
    if (kt < nk) DMPQ_F4F_ITER(0, 1)
#undef DMPQ_F4F_GLOAD
#undef DMPQ_F4F_DQ
#undef DMPQ_F4F_FRAG
#undef DMPQ_F4F_MFMA
#undef DMPQ_F4F_ITER

    fp4_epilogue<OUT, EPI>(acc, lds, ga, gw, M, N, m0, n0, wave, wm, wn, lane, y, partial, pid);
}

// One k-step fragment: the 8 codes of 32-bit word S of a 16-byte piece, times
// the piece's scale (element 0 of s2 for words 0-1, element 1 for words 2-3).
template <int S>
__device__ __forceinline__ v8h dq8(const uint4 c, const v2h s2) {
    const uint32_t w = S == 0 ? c.x : S == 1 ? c.y : S == 2 ? c.z : c.w;
    const v2h sc = S < 2 ? __builtin_shufflevector(s2, s2, 0, 0) : __builtin_shufflevector(s2, s2, 1, 1);
    const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
    const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
    const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
    const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
    return (v8h){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// ---------------------------------------------------------------------------
// DMA path (K % 128 == 0).  Raw codes and scales go from global memory
// straight into LDS with global_load_lds, and every wave dequantizes the
// fragments of its own MFMAs from LDS into registers.  Compared with staging
// dequantized tiles, the load path touches whole 128-byte row segments, and
// LDS holds 4.5 bits per element instead of 16.
//
// A stage is 256 K elements.  Per operand: 256 rows x 128 code bytes, piece
// p of a row (16 bytes = K positions 32p .. 32p+31) stored at slot
// p ^ ((row >> 1) & 7), so the 32-row fragment reads hit distinct 16-byte
// slots of each 256-byte bank span; and 256 rows x 16 scale bytes, row-major.
// Two stages in flight.  K order inside a 64-element chunk c: lane half h
// holds piece 2c + h and feeds k-step s the positions 8s .. 8s+7 of it (the
// same order on both operands, so products pair the same elements).
//
// When K % 256 == 128 (K >= 384, e.g. a 1920 hidden) the last stage is a
// half stage of 128 elements (HT), which ends 64 code bytes and 8 scale bytes
// before a full stage would.  There a lane whose piece lies in the missing
// half loads the piece 64 bytes earlier (in bounds, never read), and the
// scale DMA loads the row's 16 bytes from 8 bytes earlier, so the stage's 8
// scale bytes land in words 2 and 3 of the row's slot; the half stage runs
// chunks 0 and 1 only.
// ---------------------------------------------------------------------------
namespace fp4dma {
constexpr int BM = 256, BN = 256, BKE = 256;
constexpr int CROW = BKE / 2, SROW = BKE / 16;   // code / scale bytes per row per stage
constexpr int CODES = BM * CROW, SCALES = BM * SROW;
constexpr int STAGE = 2 * CODES + 2 * SCALES;   // A codes, W codes, A scales, W scales
constexpr int LDS_BYTES = 2 * STAGE > 4 * EpiBand<4>::BYTES ? 2 * STAGE : 4 * EpiBand<4>::BYTES;
constexpr int CBLK = CODES / 1024 / 4;          // 1 KB code blocks per wave per operand
constexpr int PER = 2 * CBLK + 2;               // DMA instructions per wave per stage
constexpr unsigned GROUP_M = 8;
static_assert(LDS_BYTES <= 160 * 1024, "LDS of the NVFP4 DMA kernels");
__device__ __forceinline__ int key(int row) { return (row >> 1) & 7; }
}  // namespace fp4dma

// Per-lane state of the DMA kernel.  Fragment rows ra = wm*128 + 32i + lane%32
// share the swizzle key of lane%32, so the row block i only adds a constant
// (an immediate offset) to the lane's base addresses.
struct Fp4DmaLane {
    // DMA sources: the tile's first rows of each operand (uniform) and the
    // lane's byte offsets from them (32-bit: 256 rows of K / 2 bytes, K <=
    // 2^22), so that an address is a scalar base plus a vector offset
    const uint8_t *ca, *cw, *sa, *sw;
    uint32_t goffA[fp4dma::CBLK], goffW[fp4dma::CBLK], goffSA, goffSW;
    int offA, offW, offSA, offSW;  // byte offsets of the lane's first fragment row in a stage
    int wave, hk, sh, swz;         // wave index (uniform), K half, scale shift, swizzle key
    int st_half, tail_shift;       // HT: index of the half stage; the lane's code shift there
};

// DMA instruction d (0 .. PER-1) of the stage st: code blocks q = d/2 of A (d
// even) and W (d odd), then the A and the W scale block (16 bytes per row).
template <bool HT>
__device__ __forceinline__ void fp4dma_one(uint8_t *dst, const Fp4DmaLane &L, int64_t st, int d) {
    using namespace fp4dma;
    typedef __attribute__((address_space(3))) void lds_void;
    if (d < 2 * CBLK) {
        const int q = d >> 1, b = L.wave + 4 * q;
        // base stays opaque here (and the offsets, through fp4dma_launder), so
        // that the address is a scalar base plus a 32-bit vector offset, with
        // no per-DMA 64-bit vector add
        const uint8_t *base = ((d & 1) ? L.cw : L.ca) + st * CROW;
        asm("" : "+s"(base));
        uint32_t off = (d & 1) ? L.goffW[q] : L.goffA[q];
        if constexpr (HT) off += st == L.st_half ? L.tail_shift : 0;
        __builtin_amdgcn_global_load_lds((const void *)(base + off), (lds_void *)(dst + (d & 1) * CODES + b * 1024),
                                         16, 0, 0);
    } else {
        const bool w = d == 2 * CBLK + 1;
        const uint8_t *base = (w ? L.sw : L.sa) + st * SROW;
        if constexpr (HT) base -= st == L.st_half ? 8 : 0;
        asm("" : "+s"(base));
        __builtin_amdgcn_global_load_lds((const void *)(base + (w ? L.goffSW : L.goffSA)),
                                         (lds_void *)(dst + 2 * CODES + w * SCALES + L.wave * 1024), 16, 0, 0);
    }
}

// Makes the lane's DMA offsets opaque values that change (in place, with no
// instruction) every stage, so that the compiler cannot hoist their 64-bit
// extension out of the main loop and must address by scalar base + offset.
__device__ __forceinline__ void fp4dma_launder(Fp4DmaLane &L) {
#pragma unroll
    for (int q = 0; q < fp4dma::CBLK; q++) asm("" : "+v"(L.goffA[q]), "+v"(L.goffW[q]));
    asm("" : "+v"(L.goffSA), "+v"(L.goffSW));
}

// One stage of the DMA kernel: run the stage held in `cur` while the DMA of
// stage st_next goes into `nxt`, its PER instructions spread over the MFMAs of
// the first 64-element chunk (one after every third MFMA) rather than issued
// in one burst.  The DMA is issued on every stage so that no branch wraps the
// MFMA code; after the last stage the caller passes a stage nobody reads
// again.  The two buffers are separate restrict parameters so that, once
// inlined, the compiler knows the stage's LDS reads cannot alias the DMA in
// flight and does not wait for it.  HALF: `cur` holds the half stage.
template <bool HT, bool HALF>
__device__ __forceinline__ void fp4dma_stage(const uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt,
                                             int64_t st_next, const Fp4DmaLane &L, v16f (&acc)[4][4]) {
    using namespace fp4dma;
    // the lane's scale words: word c holds the four scale bytes of chunk c
    // (the half stage's two chunks sit in words 2 and 3)
    uint4 sA[4], sW[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        sA[i] = *reinterpret_cast<const uint4 *>(cur + L.offSA + i * 32 * SROW);
        sW[i] = *reinterpret_cast<const uint4 *>(cur + L.offSW + i * 32 * SROW);
        if constexpr (HALF) {
            sA[i].x = sA[i].z;
            sA[i].y = sA[i].w;
            sW[i].x = sW[i].z;
            sW[i].y = sW[i].w;
        }
    }
#define DMPQ_F4D_CODES(dA, dW, c)                                                              \
    {                                                                                          \
        const int slot = ((2 * (c) + L.hk) ^ L.swz) * 16;                                      \
        _Pragma("unroll") for (int i = 0; i < 4; i++) {                                        \
            dA[i] = *reinterpret_cast<const uint4 *>(cur + L.offA + slot + i * 32 * CROW);     \
            dW[i] = *reinterpret_cast<const uint4 *>(cur + L.offW + slot + i * 32 * CROW);     \
        }                                                                                      \
    }
#define DMPQ_F4D_DQ(cA, cW, scA, scW, S, fa, fb)                                               \
    _Pragma("unroll") for (int i = 0; i < 4; i++) {                                            \
        fa[i] = dq8<S>(cA[i], scA[i]);                                                         \
        fb[i] = dq8<S>(cW[i], scW[i]);                                                         \
    }
// 16 MFMAs; with DMA (D0 >= 0) instructions D0, D0+1, ... (below PER) after
// MFMAs 2, 5, 8, 11, 14
#define DMPQ_F4D_MFMA(fa, fb, D0)                                                              \
    _Pragma("unroll") for (int i = 0; i < 4; i++)                                              \
        _Pragma("unroll") for (int j = 0; j < 4; j++) {                                        \
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0); \
            const int t = 4 * i + j;                                                           \
            if ((D0) >= 0 && t % 3 == 2 && (D0) + t / 3 < PER) fp4dma_one<HT>(nxt, L, st_next, (D0) + t / 3); \
        }
#define DMPQ_F4D_CHUNK(cA, cW, c, D0)                                                          \
    {                                                                                          \
        v2h scA[4], scW[4];                                                                    \
        _Pragma("unroll") for (int i = 0; i < 4; i++) {                                        \
            const uint32_t wa = (c) == 0 ? sA[i].x : (c) == 1 ? sA[i].y : (c) == 2 ? sA[i].z : sA[i].w; \
            const uint32_t ww = (c) == 0 ? sW[i].x : (c) == 1 ? sW[i].y : (c) == 2 ? sW[i].z : sW[i].w; \
            scA[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa >> L.sh, 1.0f, false);        \
            scW[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ww >> L.sh, 1.0f, false);        \
        }                                                                                      \
        v8h fa0[4], fb0[4], fa1[4], fb1[4];                                                    \
        DMPQ_F4D_DQ(cA, cW, scA, scW, 0, fa0, fb0)                                             \
        DMPQ_F4D_DQ(cA, cW, scA, scW, 1, fa1, fb1)                                             \
        DMPQ_F4D_MFMA(fa0, fb0, (D0))                                                          \
        DMPQ_F4D_DQ(cA, cW, scA, scW, 2, fa0, fb0)                                             \
        DMPQ_F4D_MFMA(fa1, fb1, (D0) < 0 ? -1 : (D0) + 5)                                      \
        DMPQ_F4D_DQ(cA, cW, scA, scW, 3, fa1, fb1)                                             \
        DMPQ_F4D_MFMA(fa0, fb0, (D0) < 0 ? -1 : (D0) + 10)                                     \
        DMPQ_F4D_MFMA(fa1, fb1, (D0) < 0 ? -1 : (D0) + 15)                                     \
    }
    uint4 cA0[4], cW0[4], cA1[4], cW1[4];
    DMPQ_F4D_CODES(cA0, cW0, 0)
    DMPQ_F4D_CODES(cA1, cW1, 1)
    DMPQ_F4D_CHUNK(cA0, cW0, 0, 0)
    if constexpr (!HALF) {
        DMPQ_F4D_CODES(cA0, cW0, 2)
        DMPQ_F4D_CHUNK(cA1, cW1, 1, -1)
        DMPQ_F4D_CODES(cA1, cW1, 3)
        DMPQ_F4D_CHUNK(cA0, cW0, 2, -1)
        DMPQ_F4D_CHUNK(cA1, cW1, 3, -1)
    } else {
        DMPQ_F4D_CHUNK(cA1, cW1, 1, -1)
    }
#undef DMPQ_F4D_CODES
#undef DMPQ_F4D_DQ
#undef DMPQ_F4D_MFMA
#undef DMPQ_F4D_CHUNK
}

// The main loop of the DMA kernel over stages kt0 .. kt1-1 of the tile at
// (m0, n0); on return the stage buffers are free.  HT: stage K / 256 is the
// half stage.
template <bool HT>
__device__ __forceinline__ void fp4dma_mainloop(const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa,
                                                const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw,
                                                int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                                int kt0, int kt1, uint8_t *lds, v16f (&acc)[4][4]) {
    using namespace fp4dma;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t nb = K / 16, rb = K / 2;
    const int nk = kt1 - kt0;

#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    // DMA sources.  Code block b = wave + 4q covers tile rows 8b .. 8b+7,
    // lane l filling slot l % 8 of row 8b + l / 8; the scale DMA of a wave
    // covers rows 64 wave .. +63, one lane per row.  Rows past M or N load a
    // clamped row; their outputs are never stored.
    Fp4DmaLane L;
    L.ca = ca + m0 * rb;
    L.cw = cw + n0 * rb;
    L.sa = sa + m0 * nb;
    L.sw = sw + n0 * nb;
    L.wave = wave;
    L.hk = lane >> 5;
    L.sh = 16 * L.hk;
#pragma unroll
    for (int q = 0; q < CBLK; q++) {
        const int row = 8 * (wave + 4 * q) + lane / 8;
        const int piece = (lane % 8) ^ key(row);
        const int64_t gm = m0 + row < M ? m0 + row : M - 1;
        const int64_t gn = n0 + row < N ? n0 + row : N - 1;
        L.goffA[q] = (uint32_t)((gm - m0) * rb + piece * 16);
        L.goffW[q] = (uint32_t)((gn - n0) * rb + piece * 16);
    }
    {
        const int row = 64 * wave + lane;
        const int64_t gm = m0 + row < M ? m0 + row : M - 1;
        const int64_t gn = n0 + row < N ? n0 + row : N - 1;
        L.goffSA = (uint32_t)((gm - m0) * nb);
        L.goffSW = (uint32_t)((gn - n0) * nb);
    }
    const int ra = wm * 128 + (lane & 31), rw = wn * 128 + (lane & 31);
    L.offA = ra * CROW;
    L.offW = CODES + rw * CROW;
    L.offSA = 2 * CODES + ra * SROW;
    L.offSW = 2 * CODES + SCALES + rw * SROW;
    L.swz = key(lane & 31);
    // HT: the lane's code piece is the same in every block q (key(8 (wave +
    // 4q) + lane / 8) does not depend on q); pieces 4 .. 7 lie in the half
    // stage's missing half
    L.st_half = (int)(K / 256);
    L.tail_shift = ((lane % 8) ^ key(8 * wave + lane / 8)) >= 4 ? -64 : 0;
    const bool half_last = HT && kt1 == L.st_half + 1;
    const int nfull = nk - (half_last ? 1 : 0);

#pragma unroll
    for (int d = 0; d < PER; d++) fp4dma_one<HT>(lds, L, kt0, d);
    for (int kt = 0; kt < nfull; kt++) {
        __builtin_amdgcn_s_waitcnt(0xC07F & ~0xC00F);  // vmcnt(0): this wave's loads of stage kt
        __syncthreads();                               // ... and every other wave's
        fp4dma_launder(L);
        // after the last stage the copy goes to a buffer nobody reads again
        fp4dma_stage<HT, false>(lds + (kt & 1) * STAGE, lds + ((kt & 1) ^ 1) * STAGE,
                                kt0 + (kt + 1 < nk ? kt + 1 : kt), L, acc);
    }
    if (half_last) {
        __builtin_amdgcn_s_waitcnt(0xC07F & ~0xC00F);
        __syncthreads();
        fp4dma_stage<HT, true>(lds + (nfull & 1) * STAGE, lds + ((nfull & 1) ^ 1) * STAGE, kt0 + nfull, L, acc);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F & ~0xC00F);  // the last copy has landed
    __syncthreads();  // every wave is done reading the stage buffers before they hold bands
}

template <int OUT, int EPI, bool HT>
__device__ __forceinline__ void fp4dma_tile(const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa,
                                            const float *__restrict__ ga, const uint8_t *__restrict__ cw,
                                            const uint8_t *__restrict__ sw, const float *__restrict__ gw,
                                            int64_t M, int64_t N, int64_t K, void *__restrict__ y,
                                            unsigned tiles_m, unsigned tiles_n, float *__restrict__ partial,
                                            uint8_t *lds) {
    using namespace fp4dma;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;
    v16f acc[4][4];
    fp4dma_mainloop<HT>(ca, sa, cw, sw, M, N, K, m0, n0, 0, (int)(K / BKE) + (HT ? 1 : 0), lds, acc);
    fp4_epilogue<OUT, EPI>(acc, lds, ga, gw, M, N, m0, n0, wave, wm, wn, lane, y, partial, pid);
}

// The whole-tile kernels: K % 256 == 0, and with the closing half stage
// (kernels of their own, so that each keeps its name in traces).
template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_fp4_dma_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n,
    float *__restrict__ partial) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fp4dma_tile<OUT, EPI, false>(ca, sa, ga, cw, sw, gw, M, N, K, y, tiles_m, tiles_n, partial, lds);
}

template <int OUT, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_fp4_dma_tail_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n,
    float *__restrict__ partial) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fp4dma_tile<OUT, EPI, true>(ca, sa, ga, cw, sw, gw, M, N, K, y, tiles_m, tiles_n, partial, lds);
}

// The split workgroups of a SplitPlan launch (see gemm_i8_split_kernel).
template <bool HT>
__device__ __forceinline__ void fp4dma_split(const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa,
                                             const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw,
                                             int64_t M, int64_t N, int64_t K, unsigned tiles_m, unsigned tiles_n,
                                             const SplitPlan &sp, uint32_t *__restrict__ spart,
                                             float *__restrict__ partial, uint8_t *lds) {
    using namespace fp4dma;
    const SplitUnit u = split_unit(sp, tiles_m, tiles_n, GROUP_M);
    if (partial && u.kt0 == 0 && threadIdx.x == 0) partial[sp.full + blockIdx.x / sp.splits] = 0.0f;
    v16f acc[4][4];
    fp4dma_mainloop<HT>(ca, sa, cw, sw, M, N, K, (int64_t)u.tc.m * BM, (int64_t)u.tc.n * BN, u.kt0, u.kt1, lds, acc);
    store_split_partial(acc, spart + (size_t)blockIdx.x * kSplitWords, threadIdx.x);
}

__global__ __launch_bounds__(256, 1) void gemm_fp4_split_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const uint8_t *__restrict__ cw,
    const uint8_t *__restrict__ sw, int64_t M, int64_t N, int64_t K, unsigned tiles_m, unsigned tiles_n,
    SplitPlan sp, uint32_t *__restrict__ spart, float *__restrict__ partial) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fp4dma_split<false>(ca, sa, cw, sw, M, N, K, tiles_m, tiles_n, sp, spart, partial, lds);
}

__global__ __launch_bounds__(256, 1) void gemm_fp4_split_tail_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const uint8_t *__restrict__ cw,
    const uint8_t *__restrict__ sw, int64_t M, int64_t N, int64_t K, unsigned tiles_m, unsigned tiles_n,
    SplitPlan sp, uint32_t *__restrict__ spart, float *__restrict__ partial) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    fp4dma_split<true>(ca, sa, cw, sw, M, N, K, tiles_m, tiles_n, sp, spart, partial, lds);
}

// ---------------------------------------------------------------------------
// Variant DMPQ_FP4_SCALED_MFMA: gfx950's block-scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 operands) with the NVFP4 scales
// applied exactly.  The instruction scales each 32-element K-slot by a power
// of two (E8M0), which cannot represent an E4M3 scale, and it sums the
// slots, so one 16-element group goes alone into one instruction (its codes
// in the first half of slot 0, everything else zero, E8M0 scales 2^0).  That
// yields the exact group partial P[m][n] = sum_k vA vW, which the VALU folds
// in as acc += P * (sA[m,g] * sW[n,g]) in fp32 (the scale product is exact).
// 1/4 of each MFMA's K carries data and the rescale costs two VALU ops per
// output element per group; the in-LDS dequant (variant 0) is the faster
// exact path on this chip.
//
// Tiling: 256 threads = 2 x 2 waves, workgroup tile 128 x 128, wave tile
// 64 x 64 = 2 x 2 MFMA 32x32 tiles; 8 scale groups per LDS stage (codes
// staged as bytes, scales decoded to fp32 once per workgroup).
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));

namespace fp4scaled {
constexpr int BM = 128, BN = 128, G = 8;  // G scale groups per LDS stage
}

template <int OUT>
__global__ __launch_bounds__(256) void gemm_fp4_scaled_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, void *__restrict__ y, unsigned tiles_n) {
    using namespace fp4scaled;
    // [group][row]: a lane's 8-byte fragment read is row-contiguous (no bank conflicts)
    __shared__ __attribute__((aligned(16))) uint2 codes_a[G][BM], codes_w[G][BN];
    __shared__ __attribute__((aligned(16))) float sca[G][BM], scw[G][BN];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM, n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const int64_t nb = K / 16, rb = K / 2;

    // staging role: row tid/2 of both tiles, groups 4*(tid&1) .. +3
    const int sr = tid >> 1, sg = 4 * (tid & 1);
    const int64_t gm = m0 + sr < M ? m0 + sr : M - 1;  // clamped; rows past M are never stored
    const int64_t gn = n0 + sr < N ? n0 + sr : N - 1;

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    for (int64_t g0 = 0; g0 < nb; g0 += G) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int gl = sg + q;
            const bool kin = g0 + gl < nb;
            const int64_t gi = kin ? g0 + gl : nb - 1;
            const uint2 a = *reinterpret_cast<const uint2 *>(ca + gm * rb + 8 * gi);
            const uint2 w = *reinterpret_cast<const uint2 *>(cw + gn * rb + 8 * gi);
            const float fa = e4m3_value(sa[gm * nb + gi]), fw = e4m3_value(sw[gn * nb + gi]);
            codes_a[gl][sr] = kin ? a : make_uint2(0u, 0u);
            codes_w[gl][sr] = kin ? w : make_uint2(0u, 0u);
            sca[gl][sr] = kin ? fa : 0.0f;
            scw[gl][sr] = kin ? fw : 0.0f;
        }
        __syncthreads();
#pragma unroll 2
        for (int gl = 0; gl < G; gl++) {
            v8i fa[2], fb[2];
            float s_a[2][16], s_w[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const int ra = wm * 64 + i * 32 + (lane & 31);
                const int rw = wn * 64 + i * 32 + (lane & 31);
                // lanes 32..63 carry K positions 32..63 of the instruction: zero
                const uint2 a = codes_a[gl][ra], w = codes_w[gl][rw];
                const bool lo = lane < 32;
                fa[i] = (v8i){lo ? (int)a.x : 0, lo ? (int)a.y : 0, 0, 0, 0, 0, 0, 0};
                fb[i] = (v8i){lo ? (int)w.x : 0, lo ? (int)w.y : 0, 0, 0, 0, 0, 0, 0};
                s_w[i] = scw[gl][rw];
#pragma unroll
                for (int r4 = 0; r4 < 4; r4++) {
                    const float4 v = *reinterpret_cast<const float4 *>(
                        &sca[gl][wm * 64 + i * 32 + 8 * r4 + 4 * (lane >> 5)]);
                    s_a[i][4 * r4 + 0] = v.x;
                    s_a[i][4 * r4 + 1] = v.y;
                    s_a[i][4 * r4 + 2] = v.z;
                    s_a[i][4 * r4 + 3] = v.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 2; i++) {
#pragma unroll
                for (int j = 0; j < 2; j++) {
                    const v16f zero = {};
                    // format 4 = E2M1 for both operands, E8M0 scales 127 = 2^0
                    const v16f p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], zero, 4, 4, 0, 127, 0, 127);
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        // p (<= 576, a multiple of 1/4) times an E4M3 x E4M3 product
                        // is exact in fp32, so the fused multiply-add rounds once,
                        // exactly like a separate multiply and add would
                        acc[i][j][r] = __builtin_fmaf(p[r], s_a[i][r] * s_w[j], acc[i][j][r]);
                    }
                }
            }
        }
    }

    const float gA = *ga, gW = *gw;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const float v = (acc[i][j][r] * gA) * gW;
                if constexpr (OUT == 0)
                    static_cast<float *>(y)[row * N + col] = v;
                else
                    static_cast<uint16_t *>(y)[row * N + col] = (uint16_t)f32_to_bf16(v);
            }
        }
}

template <class KernelFn>
static hipError_t allow_lds(KernelFn fn, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// The DMA path: the whole-tile kernel over the full waves, then (with a split
// plan) the tail's split workgroups and the fixup.  HT: K / 256 full stages
// and the half stage.
template <int OUT, int EPI, bool HT, class TileFn, class SplitFn>
static hipError_t launch_fp4_dma(hipStream_t s, TileFn tile_kernel, SplitFn split_kernel, const uint8_t *ca,
                                 const uint8_t *sa, const float *ga, const uint8_t *cw, const uint8_t *sw,
                                 const float *gw, int64_t M, int64_t N, int64_t K, void *y, float *partial,
                                 uint32_t *spart, unsigned utm, unsigned utn) {
    const SplitPlan sp = plan_split((int64_t)utm * utn, (int)(K / fp4dma::BKE) + (HT ? 1 : 0), spart != nullptr);
    if (sp.full > 0) {
        hipLaunchKernelGGL(tile_kernel, dim3(sp.full), dim3(256), fp4dma::LDS_BYTES, s, ca, sa, ga, cw, sw, gw, M,
                           N, K, y, utm, utn, partial);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sp.splits > 1) {
        hipLaunchKernelGGL(split_kernel, dim3(sp.tail * sp.splits), dim3(256), fp4dma::LDS_BYTES, s, ca, sa, cw, sw,
                           M, N, K, utm, utn, sp, spart, (EPI & kEpiAmax) ? partial : nullptr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_f32_fixup(s, ga, gw, M, N, y, utm, utn, fp4dma::GROUP_M, partial, sp, spart, OUT, EPI);
    }
    return hipGetLastError();
}

template <int OUT, int EPI>
static hipError_t launch_fp4_paths(hipStream_t s, const uint8_t *ca, const uint8_t *sa,
                                   const float *ga, const uint8_t *cw, const uint8_t *sw,
                                   const float *gw, int64_t M, int64_t N, int64_t K, void *y,
                                   float *partial, uint32_t *spart) {
    using namespace fp4gemm;
    static const hipError_t attr = [] {
        hipError_t e = allow_lds(gemm_fp4_f16_kernel<OUT, EPI>, 2 * STAGE);
        if (e == hipSuccess) e = allow_lds(gemm_fp4_fast_kernel<OUT, EPI>, 2 * STAGE);
        if (e == hipSuccess) e = allow_lds(gemm_fp4_dma_kernel<OUT, EPI>, fp4dma::LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_fp4_split_kernel, fp4dma::LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_fp4_dma_tail_kernel<OUT, EPI>, fp4dma::LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_fp4_split_tail_kernel, fp4dma::LDS_BYTES);
        return e;
    }();
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tm * tn)), block(256);
    const unsigned utm = (unsigned)tm, utn = (unsigned)tn;
    if (K % 256 == 0)
        return launch_fp4_dma<OUT, EPI, false>(s, gemm_fp4_dma_kernel<OUT, EPI>, gemm_fp4_split_kernel, ca, sa, ga,
                                               cw, sw, gw, M, N, K, y, partial, spart, utm, utn);
    if (K % 128 == 0 && K >= 384)
        return launch_fp4_dma<OUT, EPI, true>(s, gemm_fp4_dma_tail_kernel<OUT, EPI>, gemm_fp4_split_tail_kernel, ca,
                                              sa, ga, cw, sw, gw, M, N, K, y, partial, spart, utm, utn);
    if (K % (4 * 16) == 0) {
        hipLaunchKernelGGL((gemm_fp4_fast_kernel<OUT, EPI>), grid, block, 2 * STAGE, s, ca, sa, ga, cw,
                           sw, gw, M, N, K, y, utm, utn, partial);
    } else {
        hipLaunchKernelGGL((gemm_fp4_f16_kernel<OUT, EPI>), grid, block, 2 * STAGE, s, ca, sa, ga, cw,
                           sw, gw, M, N, K, y, utm, utn, partial);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_nvfp4(hipStream_t s, const uint8_t *ca, const uint8_t *sa,
                             const float *ga, const uint8_t *cw, const uint8_t *sw,
                             const float *gw, int64_t M, int64_t N, int64_t K, int out_dtype,
                             void *y, int variant, int epi, float *partial, uint32_t *spart) {
    if (M == 0 || N == 0) return hipSuccess;
    if (variant == 1) {
        if (epi != 0) return hipErrorInvalidValue;
        const int64_t sm = (M + fp4scaled::BM - 1) / fp4scaled::BM, sn = (N + fp4scaled::BN - 1) / fp4scaled::BN;
        const dim3 block(256);
        if (out_dtype == 0)
            hipLaunchKernelGGL(gemm_fp4_scaled_kernel<0>, dim3((unsigned)(sm * sn)), block, 0, s, ca, sa, ga, cw, sw, gw, M, N, K, y, (unsigned)sn);
        else
            hipLaunchKernelGGL(gemm_fp4_scaled_kernel<1>, dim3((unsigned)(sm * sn)), block, 0, s, ca, sa, ga, cw, sw, gw, M, N, K, y, (unsigned)sn);
        return hipGetLastError();
    }
    if (out_dtype == 0 && epi == 0)
        return launch_fp4_paths<0, 0>(s, ca, sa, ga, cw, sw, gw, M, N, K, y, partial, spart);
    if (out_dtype != 1) return hipErrorInvalidValue;
    switch (epi) {
        case 0: return launch_fp4_paths<1, 0>(s, ca, sa, ga, cw, sw, gw, M, N, K, y, partial, spart);
        case 1: return launch_fp4_paths<1, 1>(s, ca, sa, ga, cw, sw, gw, M, N, K, y, partial, spart);
        case 2: return launch_fp4_paths<1, 2>(s, ca, sa, ga, cw, sw, gw, M, N, K, y, partial, spart);
        case 3: return launch_fp4_paths<1, 3>(s, ca, sa, ga, cw, sw, gw, M, N, K, y, partial, spart);
    }
    return hipErrorInvalidValue;
}

}  // namespace dmpq
