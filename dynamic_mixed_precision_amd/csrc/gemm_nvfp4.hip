// gemm_nvfp4.hip -- NVFP4 quantized linear on gfx950.  Method: 6Bit-Diffusion
// routes temporally stable layers to NVFP4 (E2M1 elements, one E4M3 scale
// per 16, an fp32 tensor scale) against NVFP4 weights (gist.science
// summaries §1 and §2.A).
//
// gfx950's block-scaled MFMA takes one power-of-two (E8M0) scale per 32
// elements, which cannot carry an E4M3 scale per 16 exactly.  This kernel
// instead dequantizes exactly: an E2M1 value (<= 2 significant bits) times an
// E4M3 scale (<= 4 significant bits) has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in bf16.  The bf16 MFMA products are exact
// in fp32; only the fp32 accumulation rounds.  y = (acc * gA) * gW.
//
// Tiling: 256 threads = 2 x 2 waves, workgroup tile 128 x 128, wave tile
// 64 x 64 = 2 x 2 MFMA 32x32x16 tiles, 64 k-elements (4 scale groups) per
// LDS stage, each thread dequantizing two 16-element groups per operand.
#include "device.hpp"
#include "internal.hpp"

namespace dmpq {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

namespace {
constexpr int BM = 128, BN = 128, BKE = 64;
constexpr int LDS_ROW = BKE * 2 + 16;  // bytes per staged row (bf16 + pad)

// E2M1 code (4 bits) -> fp32 value.
__device__ __forceinline__ float e2m1_f32(uint32_t code) {
    const uint32_t mag = code & 7u;
    const uint32_t bits = mag >= 2u ? ((((mag >> 1) + 126u) << 23) | ((mag & 1u) << 22))
                                    : (mag ? 0x3F000000u : 0u);
    return __uint_as_float(bits | ((code & 8u) << 28));
}

// 16 codes (8 bytes) with one E4M3 scale -> 16 bf16 (exact), as 8 words.
__device__ __forceinline__ void dequant16(uint2 c, uint32_t scale_code, uint32_t out[8]) {
    const float s = e4m3_value(scale_code);
    const uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const float lo = e2m1_f32(byte & 15u) * s;
        const float hi = e2m1_f32(byte >> 4) * s;
        out[i] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
    }
}
}  // namespace

__global__ __launch_bounds__(256) void gemm_fp4_bf16_kernel(
    const uint8_t *__restrict__ ca, const uint8_t *__restrict__ sa, const float *__restrict__ ga,
    const uint8_t *__restrict__ cw, const uint8_t *__restrict__ sw, const float *__restrict__ gw,
    int64_t M, int64_t N, int64_t K, int out_dtype, void *__restrict__ y, unsigned tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t As[BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) uint8_t Ws[BN * LDS_ROW];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;
    const int64_t nb = K / 16;

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

    // thread -> (row, pair of 16-groups) of the stage
    const int lrow = tid >> 1, lhalf = tid & 1;
    uint2 rca[2], rcw[2];
    uint32_t rsa[2], rsw[2];
    auto gload = [&](int64_t g0) {  // g0: first scale group of the stage
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int64_t gi = g0 + 2 * lhalf + h;
            const int64_t gm = m0 + lrow, gn = n0 + lrow;
            const bool ka = gi < nb;
            rca[h] = (ka && gm < M) ? *reinterpret_cast<const uint2 *>(ca + gm * (K / 2) + 8 * gi)
                                    : make_uint2(0u, 0u);
            rsa[h] = (ka && gm < M) ? sa[gm * nb + gi] : 0u;
            rcw[h] = (ka && gn < N) ? *reinterpret_cast<const uint2 *>(cw + gn * (K / 2) + 8 * gi)
                                    : make_uint2(0u, 0u);
            rsw[h] = (ka && gn < N) ? sw[gn * nb + gi] : 0u;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int h = 0; h < 2; h++) {
            uint32_t d[8];
            const int off = lrow * LDS_ROW + (2 * lhalf + h) * 32;
            dequant16(rca[h], rsa[h], d);
            *reinterpret_cast<uint4 *>(As + off) = make_uint4(d[0], d[1], d[2], d[3]);
            *reinterpret_cast<uint4 *>(As + off + 16) = make_uint4(d[4], d[5], d[6], d[7]);
            dequant16(rcw[h], rsw[h], d);
            *reinterpret_cast<uint4 *>(Ws + off) = make_uint4(d[0], d[1], d[2], d[3]);
            *reinterpret_cast<uint4 *>(Ws + off + 16) = make_uint4(d[4], d[5], d[6], d[7]);
        }
    };

    gload(0);
    for (int64_t g0 = 0; g0 < nb; g0 += BKE / 16) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (g0 + BKE / 16 < nb) gload(g0 + BKE / 16);
#pragma unroll
        for (int ks = 0; ks < BKE; ks += 16) {
            v8bf a[2], b[2];
            const int koff = (ks + 8 * (lane >> 5)) * 2;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                a[i] = *reinterpret_cast<const v8bf *>(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_ROW + koff);
                b[i] = *reinterpret_cast<const v8bf *>(Ws + (wn * 64 + i * 32 + (lane & 31)) * LDS_ROW + koff);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    const float gA = *ga, gW = *gw;
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const float v = (acc[i][j][r] * gA) * gW;
                const int64_t o = row * N + col;
                if (out_dtype == 0)
                    static_cast<float *>(y)[o] = v;
                else
                    static_cast<uint16_t *>(y)[o] = (uint16_t)f32_to_bf16(v);
            }
        }
    }
}

hipError_t launch_gemm_nvfp4(hipStream_t s, const uint8_t *ca, const uint8_t *sa,
                             const float *ga, const uint8_t *cw, const uint8_t *sw,
                             const float *gw, int64_t M, int64_t N, int64_t K, int out_dtype,
                             void *y, int variant) {
    (void)variant;
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_fp4_bf16_kernel, dim3((unsigned)(tm * tn)), dim3(256), 0, s, ca, sa,
                       ga, cw, sw, gw, M, N, K, out_dtype, y, (unsigned)tn);
    return hipGetLastError();
}

}  // namespace dmpq
