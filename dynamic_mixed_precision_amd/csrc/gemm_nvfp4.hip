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
    // stage (16 code bytes = 32 elements = 2 scale groups)
    uint4 rca[2], rcw[2];
    uint32_t rsa[2], rsw[2];
    const int nk = (int)((nb + 3) / 4);

    // Out-of-range chunks read a clamped in-range address and are replaced by
    // zero codes / zero scales (a value select; no pointer to a local).
#define DMPQ_F4_GLOAD(g0)                                                                     \
    _Pragma("unroll") for (int h = 0; h < 2; h++) {                                           \
        const int c = tid + 256 * h;                                                          \
        const int r = c >> 1;                                                                 \
        const int64_t gi = (g0) + 2 * (c & 1); /* first scale group of the chunk */           \
        const int64_t gic = gi < nb ? gi : nb - 1;                                            \
        const int64_t gm = m0 + r, gn = n0 + r;                                               \
        const int64_t gmc = gm < M ? gm : M - 1, gnc = gn < N ? gn : N - 1;                   \
        const uint2 a0 = *reinterpret_cast<const uint2 *>(ca + gmc * rb + 8 * gic);           \
        const uint2 w0 = *reinterpret_cast<const uint2 *>(cw + gnc * rb + 8 * gic);           \
        const int64_t gic1 = gi + 1 < nb ? gi + 1 : nb - 1;                                   \
        const uint2 a1 = *reinterpret_cast<const uint2 *>(ca + gmc * rb + 8 * gic1);          \
        const uint2 w1 = *reinterpret_cast<const uint2 *>(cw + gnc * rb + 8 * gic1);          \
        const uint32_t sa0 = sa[gmc * nb + gic], sa1 = sa[gmc * nb + gic1];                   \
        const uint32_t sw0 = sw[gnc * nb + gic], sw1 = sw[gnc * nb + gic1];                   \
        const bool a_ok0 = gm < M && gi < nb, a_ok1 = gm < M && gi + 1 < nb;                  \
        const bool w_ok0 = gn < N && gi < nb, w_ok1 = gn < N && gi + 1 < nb;                  \
        rca[h] = make_uint4(a_ok0 ? a0.x : 0u, a_ok0 ? a0.y : 0u, a_ok1 ? a1.x : 0u, a_ok1 ? a1.y : 0u); \
        rcw[h] = make_uint4(w_ok0 ? w0.x : 0u, w_ok0 ? w0.y : 0u, w_ok1 ? w1.x : 0u, w_ok1 ? w1.y : 0u); \
        rsa[h] = (a_ok0 ? sa0 : 0u) | ((a_ok1 ? sa1 : 0u) << 8);                              \
        rsw[h] = (w_ok0 ? sw0 : 0u) | ((w_ok1 ? sw1 : 0u) << 8);                              \
    }
#define DMPQ_F4_SSTORE(buf)                                                                   \
    _Pragma("unroll") for (int h = 0; h < 2; h++) {                                           \
        const int c = tid + 256 * h;                                                          \
        const int r = c >> 1;                                                                 \
        uint8_t *pa = lds + (buf) * STAGE + r * ROW + (c & 1) * 64;                           \
        uint8_t *pw = lds + (buf) * STAGE + (BM + r) * ROW + (c & 1) * 64;                    \
        uint32_t d[16];                                                                       \
        dequant32(rca[h], rsa[h], d);                                                         \
        _Pragma("unroll") for (int q = 0; q < 4; q++)                                         \
            *reinterpret_cast<uint4 *>(pa + 16 * q) = make_uint4(d[4 * q], d[4 * q + 1], d[4 * q + 2], d[4 * q + 3]); \
        dequant32(rcw[h], rsw[h], d);                                                         \
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
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            DMPQ_F4_SSTORE(cur ^ 1)
        }
        __syncthreads();
    }
#undef DMPQ_F4_GLOAD
#undef DMPQ_F4_SSTORE

    const float gA = *ga, gW = *gw;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
        if (col >= N) continue;
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const float v = (acc[i][j][r] * gA) * gW;
                const int64_t o = row * N + col;
                if constexpr (OUT == 0)
                    static_cast<float *>(y)[o] = v;
                else
                    static_cast<uint16_t *>(y)[o] = (uint16_t)f32_to_bf16(v);
            }
        }
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
