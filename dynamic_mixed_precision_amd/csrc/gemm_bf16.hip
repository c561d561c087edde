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

template <int OUT, bool TAIL>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t M, int64_t N,
    int64_t K, void *__restrict__ y, unsigned tiles_m, unsigned tiles_n) {
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
    f32_band_epilogue<OUT>(acc, lds, 1.0f, 1.0f, M, N, m0, n0, wave, wm, wn, lane, y);
}

template <class KernelFn>
static hipError_t allow_lds(KernelFn fn, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_gemm_bf16(hipStream_t s, const uint16_t *x, const uint16_t *w, int64_t M,
                            int64_t N, int64_t K, int out_dtype, void *y) {
    using namespace gdma;
    if (M == 0 || N == 0) return hipSuccess;
    static const hipError_t attr = [] {
        hipError_t e = allow_lds(gemm_bf16_kernel<0, false>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_kernel<1, false>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_kernel<0, true>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_kernel<1, true>, LDS_BYTES);
        return e;
    }();
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tm * tn)), block(256);
    const unsigned utm = (unsigned)tm, utn = (unsigned)tn;
    const bool tail = (2 * K) % BK != 0;
    if (!tail && out_dtype == 0)
        hipLaunchKernelGGL((gemm_bf16_kernel<0, false>), grid, block, LDS_BYTES, s, x, w, M, N, K, y, utm, utn);
    else if (!tail)
        hipLaunchKernelGGL((gemm_bf16_kernel<1, false>), grid, block, LDS_BYTES, s, x, w, M, N, K, y, utm, utn);
    else if (out_dtype == 0)
        hipLaunchKernelGGL((gemm_bf16_kernel<0, true>), grid, block, LDS_BYTES, s, x, w, M, N, K, y, utm, utn);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<1, true>), grid, block, LDS_BYTES, s, x, w, M, N, K, y, utm, utn);
    return hipGetLastError();
}

}  // namespace dmpq
