// gemm_bf16.hip -- the full-precision linear of the Purified Delta Refresh
// route: y = x w^T over bf16 operands with fp32 accumulation, no quantization.
// Method: 6Bit-Diffusion computes a block in full precision (FP16/BF16) on a
// refresh step whose input has a high outlier ratio, so the delta written to
// the cache carries no quantization noise (gist.science summaries, §2.C).
//
// The DMA-fed main loop of gemm_dma.hpp with v_mfma_f32_32x32x16_bf16: a
// stage is 64 bf16 values of every row.  K % 64 != 0 takes the TAIL form of
// the loop (the partial last stage's k-steps past K read as zeros).  The bf16
// products are exact in fp32; only the fp32 accumulation rounds.
#include "device.hpp"
#include "gemm_common.hpp"
#include "gemm_dma.hpp"
#include "internal.hpp"

namespace dmpq {

template <int OUT, bool TAIL, int EPI>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t M, int64_t N,
    int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n, float *__restrict__ partial) {
    using namespace gdma;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const TileCoord tc = tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;

    v16f acc[4][4];
    dma_gemm_mainloop<OpBF16, TAIL>(reinterpret_cast<const uint8_t *>(x),
                                    reinterpret_cast<const uint8_t *>(w), M, N, 2 * K, m0, n0,
                                    lds, acc);
    f32_band_epilogue<OUT, EPI>(acc, lds, 1.0f, 1.0f, M, N, m0, n0, wave, wm, wn, lane, y, partial);
}

template <class KernelFn>
static hipError_t allow_lds(KernelFn fn, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int OUT, int EPI>
static hipError_t launch_bf16_paths(hipStream_t s, const uint16_t *x, const uint16_t *w, int64_t M,
                                    int64_t N, int64_t K, void *y, float *partial) {
    using namespace gdma;
    static const hipError_t attr = [] {
        hipError_t e = allow_lds(gemm_bf16_kernel<OUT, false, EPI>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_kernel<OUT, true, EPI>, LDS_BYTES);
        return e;
    }();
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tm * tn)), block(256);
    const unsigned utm = (unsigned)tm, utn = (unsigned)tn;
    if ((2 * K) % BK == 0)
        hipLaunchKernelGGL((gemm_bf16_kernel<OUT, false, EPI>), grid, block, LDS_BYTES, s, x, w, M, N, K, y,
                           utm, utn, partial);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<OUT, true, EPI>), grid, block, LDS_BYTES, s, x, w, M, N, K, y,
                           utm, utn, partial);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(hipStream_t s, const uint16_t *x, const uint16_t *w, int64_t M,
                            int64_t N, int64_t K, int out_dtype, void *y, int epi, float *partial) {
    if (M == 0 || N == 0) return hipSuccess;
    if (out_dtype == 0 && epi == 0) return launch_bf16_paths<0, 0>(s, x, w, M, N, K, y, partial);
    if (out_dtype != 1) return hipErrorInvalidValue;
    switch (epi) {
        case 0: return launch_bf16_paths<1, 0>(s, x, w, M, N, K, y, partial);
        case 1: return launch_bf16_paths<1, 1>(s, x, w, M, N, K, y, partial);
        case 2: return launch_bf16_paths<1, 2>(s, x, w, M, N, K, y, partial);
        case 3: return launch_bf16_paths<1, 3>(s, x, w, M, N, K, y, partial);
    }
    return hipErrorInvalidValue;
}

}  // namespace dmpq
