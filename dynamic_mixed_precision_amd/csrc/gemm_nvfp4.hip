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
// block's scale.  The dequantized tiles go to LDS once per workgroup.
//
// Tiling: 256 threads = 2 x 2 waves, workgroup tile 256 x 256, wave tile
// 128 x 128 = 4 x 4 MFMA 32x32x16 tiles.  K advances 64 elements (4 scale
// groups) per stage through a double-buffered LDS (fp16 rows of 128 bytes
// padded to 144); the next stage's codes and scales are in flight during the
// current stage's MFMAs.
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

template <int OUT>
__global__ __launch_bounds__(256, 1) void gemm_fp4_f16_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n) {
    using namespace fp4gemm;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const TileCoord tc = tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, GROUP_M);
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

    // staging: chunk c = tid + 256*h (h = 0, 1) is row c/2, k-half c%2 of the
    // stage (16 code bytes = 32 elements = 2 scale groups).  Out-of-range
    // groups read a clamped in-range address; bits of `ok` record which groups
    // are real and the zeroing is applied when the chunk is dequantized into
    // LDS, after the stage's MFMAs have been issued.
    uint2 rca[2][2], rcw[2][2];
    uint32_t rsa[2][2], rsw[2][2];
    uint32_t ok = 0u;  // bit 4h+q: A group q (0,1), W group q (2,3) of chunk h
    const int nk = (int)((nb + 3) / 4);

#define DMPQ_F4_GLOAD(g0)                                                                     \
    ok = 0u;                                                                                  \
    _Pragma("unroll") for (int h = 0; h < 2; h++) {                                           \
        const int c = tid + 256 * h;                                                          \
        const int r = c >> 1;                                                                 \
        const int64_t gm = m0 + r, gn = n0 + r;                                               \
        const int64_t gmc = gm < M ? gm : M - 1, gnc = gn < N ? gn : N - 1;                   \
        _Pragma("unroll") for (int q = 0; q < 2; q++) {                                       \
            const int64_t gi = (g0) + 2 * (c & 1) + q;                                        \
            const int64_t gic = gi < nb ? gi : nb - 1;                                        \
            rca[h][q] = *reinterpret_cast<const uint2 *>(ca + gmc * rb + 8 * gic);            \
            rcw[h][q] = *reinterpret_cast<const uint2 *>(cw + gnc * rb + 8 * gic);            \
            rsa[h][q] = sa[gmc * nb + gic];                                                   \
            rsw[h][q] = sw[gnc * nb + gic];                                                   \
            ok |= (uint32_t)(gm < M && gi < nb) << (4 * h + q);                               \
            ok |= (uint32_t)(gn < N && gi < nb) << (4 * h + 2 + q);                           \
        }                                                                                     \
    }
#define DMPQ_F4_SSTORE(buf)                                                                   \
    _Pragma("unroll") for (int h = 0; h < 2; h++) {                                           \
        const int c = tid + 256 * h;                                                          \
        const int r = c >> 1;                                                                 \
        uint8_t *pa = lds + (buf) * STAGE + r * ROW + (c & 1) * 64;                           \
        uint8_t *pw = lds + (buf) * STAGE + (BM + r) * ROW + (c & 1) * 64;                    \
        const bool a0 = (ok >> (4 * h)) & 1u, a1 = (ok >> (4 * h + 1)) & 1u;                  \
        const bool w0 = (ok >> (4 * h + 2)) & 1u, w1 = (ok >> (4 * h + 3)) & 1u;              \
        uint32_t d[16];                                                                       \
        dequant32(make_uint4(a0 ? rca[h][0].x : 0u, a0 ? rca[h][0].y : 0u,                    \
                             a1 ? rca[h][1].x : 0u, a1 ? rca[h][1].y : 0u),                   \
                  (a0 ? rsa[h][0] : 0u) | ((a1 ? rsa[h][1] : 0u) << 8), d);                   \
        _Pragma("unroll") for (int q = 0; q < 4; q++)                                         \
            *reinterpret_cast<uint4 *>(pa + 16 * q) = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]); \
        dequant32(make_uint4(w0 ? rcw[h][0].x : 0u, w0 ? rcw[h][0].y : 0u,                    \
                             w1 ? rcw[h][1].x : 0u, w1 ? rcw[h][1].y : 0u),                   \
                  (w0 ? rsw[h][0] : 0u) | ((w1 ? rsw[h][1] : 0u) << 8), d);                   \
        _Pragma("unroll") for (int q = 0; q < 4; q++)                                         \
            *reinterpret_cast<uint4 *>(pw + 16 * q) = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]); \
    }

    DMPQ_F4_GLOAD(0)
    DMPQ_F4_SSTORE(0)
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            DMPQ_F4_GLOAD((int64_t)(kt + 1) * 4)
        }
        const uint8_t *As = lds + cur * STAGE + (wm * 128 + (lane & 31)) * ROW + (lane >> 5) * 16;
        const uint8_t *Ws = lds + cur * STAGE + (BM + wn * 128 + (lane & 31)) * ROW + (lane >> 5) * 16;
#pragma unroll
        for (int ks = 0; ks < BKE * 2; ks += 32) {  // 16 k-elements = 32 bytes per step
            v8h a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                a[i] = *reinterpret_cast<const v8h *>(As + i * 32 * ROW + ks);
                b[i] = *reinterpret_cast<const v8h *>(Ws + i * 32 * ROW + ks);
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[j], a[i], acc[i][j], 0, 0, 0);
        }
        if (more) {
            DMPQ_F4_SSTORE(cur ^ 1)
        }
        __syncthreads();
    }
#undef DMPQ_F4_GLOAD
#undef DMPQ_F4_SSTORE

    // Epilogue (operands swapped as in the INT8 GEMM): lane l owns activation
    // row m = l % 32 of A-subtile i and four consecutive output columns
    // 8g + 4*(l/32) + 0..3 of W-subtile j per register group g.  Staged per
    // wave through LDS in two 64-row bands and stored row-contiguous.
    constexpr int ES = OUT == 1 ? 2 : 4;
    using Band = EpiBand<ES>;
    const float gA = *ga, gW = *gw;
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
                        *reinterpret_cast<uint2 *>(dst) = make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
                }
            }
        }
        epi_band_to_global<ES>(band, y, M, N, m0 + wm * 128 + h * 64, n0 + wn * 128, lane, vec);
    }
}

template <class KernelFn>
static hipError_t allow_lds(KernelFn fn, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_gemm_nvfp4(hipStream_t s, const uint8_t *ca, const uint8_t *sa,
                             const float *ga, const uint8_t *cw, const uint8_t *sw,
                             const float *gw, int64_t M, int64_t N, int64_t K, int out_dtype,
                             void *y, int variant) {
    using namespace fp4gemm;
    (void)variant;
    if (M == 0 || N == 0) return hipSuccess;
    static const hipError_t attr = [] {
        hipError_t e = allow_lds(gemm_fp4_f16_kernel<0>, 2 * STAGE);
        return e != hipSuccess ? e : allow_lds(gemm_fp4_f16_kernel<1>, 2 * STAGE);
    }();
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tm * tn)), block(256);
    if (out_dtype == 0)
        hipLaunchKernelGGL(gemm_fp4_f16_kernel<0>, grid, block, 2 * STAGE, s, ca, sa, ga, cw, sw,
                           gw, M, N, K, y, (unsigned)tm, (unsigned)tn);
    else
        hipLaunchKernelGGL(gemm_fp4_f16_kernel<1>, grid, block, 2 * STAGE, s, ca, sa, ga, cw, sw,
                           gw, M, N, K, y, (unsigned)tm, (unsigned)tn);
    return hipGetLastError();
}

}  // namespace dmpq
