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
    const unsigned pid = xcd_order(blockIdx.x, gridDim.x);
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;

    v16f acc[4][4];
    dma_gemm_mainloop<OpBF16, TAIL>(reinterpret_cast<const uint8_t *>(x),
                                    reinterpret_cast<const uint8_t *>(w), M, N, 2 * K, 2 * K, m0, n0,
                                    lds, acc);
    f32_band_epilogue<OUT, EPI>(acc, lds, 1.0f, 1.0f, M, N, m0, n0, wave, wm, wn, lane, y,
                                (EPI & kEpiAmax) ? partial + pid : nullptr);
}

// The split workgroups of a SplitPlan launch (see gemm_i8_split_kernel); the
// last split's range ends with the partial stage of a K tail.
template <bool TAIL>
__global__ __launch_bounds__(256, 1) void gemm_bf16_split_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int64_t M, int64_t N, int64_t K,
    unsigned tiles_m, unsigned tiles_n, SplitPlan sp, uint32_t *__restrict__ spart,
    float *__restrict__ partial) {
    using namespace gdma;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const SplitUnit u = split_unit(sp, tiles_m, tiles_n, GROUP_M);
    if (partial && u.kt0 == 0 && threadIdx.x == 0) partial[sp.full + blockIdx.x / sp.splits] = 0.0f;
    const int64_t k0 = (int64_t)u.kt0 * BK, k1 = (int64_t)u.kt1 * BK < 2 * K ? (int64_t)u.kt1 * BK : 2 * K;
    v16f acc[4][4];
    dma_gemm_mainloop<OpBF16, TAIL>(reinterpret_cast<const uint8_t *>(x) + k0,
                                    reinterpret_cast<const uint8_t *>(w) + k0, M, N, 2 * K, k1 - k0,
                                    (int64_t)u.tc.m * BM, (int64_t)u.tc.n * BN, lds, acc);
    store_split_partial(acc, spart + (size_t)blockIdx.x * kSplitWords, threadIdx.x);
}

// The tail tiles of a split launch with fp32 accumulators (BF16 and NVFP4
// GEMMs): one wave per 32-row slice of a 128 x 128 quadrant (16 per tail
// tile), the partials added in split order, then the fp32 epilogue.
template <int OUT, int EPI, int S>
__global__ __launch_bounds__(64) void gemm_f32_fixup_kernel(
    const float *__restrict__ ga, const float *__restrict__ gw, int64_t M, int64_t N,
    void *__restrict__ y, unsigned tiles_m, unsigned tiles_n, unsigned group_m,
    float *__restrict__ partial, SplitPlan sp, const uint32_t *__restrict__ spart) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    // workgroup = (tail tile t, quadrant wave, 32-row slice i)
    const int lane = threadIdx.x, i = blockIdx.x & 3, wave = (blockIdx.x >> 2) & 3;
    const unsigned t = blockIdx.x >> 4, pid = sp.full + t;
    const TileCoord tc = tile_at(pid, tiles_m, tiles_n, group_m);
    const int64_t m0 = (int64_t)tc.m * 256, n0 = (int64_t)tc.n * 256;
    EpiScaleF32 sc{ga ? *ga : 1.0f, gw ? *gw : 1.0f};
    split_fixup_epilogue<OUT, EPI, float, S>(spart + (size_t)t * S * kSplitWords, sc, lds, M, N, m0, n0, wave,
                                             i, lane, y, (EPI & kEpiAmax) ? partial + pid : nullptr);
}

template <class KernelFn>
static hipError_t allow_lds(KernelFn fn, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void *>(fn),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int OUT, int EPI>
static hipError_t launch_fixup(hipStream_t s, const float *ga, const float *gw, int64_t M, int64_t N,
                               void *y, unsigned tiles_m, unsigned tiles_n, unsigned group_m,
                               float *partial, const SplitPlan &sp, const uint32_t *spart) {
    const dim3 fg(16 * sp.tail), fb(64);
    const size_t fl = (size_t)kFixupRows * EpiBand<OUT == 1 ? 2 : 4>::STRIDE;
#define DMPQ_F32_FIX(S_)                                                                         \
    case S_:                                                                                     \
        hipLaunchKernelGGL((gemm_f32_fixup_kernel<OUT, EPI, S_>), fg, fb, fl, s, ga, gw, M, N, y, tiles_m, \
                           tiles_n, group_m, partial, sp, spart);                                \
        break;
    switch (sp.splits) {
        DMPQ_F32_FIX(2) DMPQ_F32_FIX(3) DMPQ_F32_FIX(4) DMPQ_F32_FIX(8)
        default: return hipErrorInvalidValue;
    }
#undef DMPQ_F32_FIX
    return hipGetLastError();
}

hipError_t launch_f32_fixup(hipStream_t s, const float *ga, const float *gw, int64_t M, int64_t N,
                            void *y, unsigned tiles_m, unsigned tiles_n, unsigned group_m,
                            float *partial, const SplitPlan &sp, const uint32_t *spart,
                            int out_dtype, int epi) {
    if (out_dtype == 0 && epi == 0)
        return launch_fixup<0, 0>(s, ga, gw, M, N, y, tiles_m, tiles_n, group_m, partial, sp, spart);
    if (out_dtype != 1) return hipErrorInvalidValue;
    switch (epi) {
        case 0: return launch_fixup<1, 0>(s, ga, gw, M, N, y, tiles_m, tiles_n, group_m, partial, sp, spart);
        case 1: return launch_fixup<1, 1>(s, ga, gw, M, N, y, tiles_m, tiles_n, group_m, partial, sp, spart);
        case 2: return launch_fixup<1, 2>(s, ga, gw, M, N, y, tiles_m, tiles_n, group_m, partial, sp, spart);
        case 3: return launch_fixup<1, 3>(s, ga, gw, M, N, y, tiles_m, tiles_n, group_m, partial, sp, spart);
    }
    return hipErrorInvalidValue;
}

template <int OUT, int EPI>
static hipError_t launch_bf16_paths(hipStream_t s, const uint16_t *x, const uint16_t *w, int64_t M,
                                    int64_t N, int64_t K, void *y, float *partial, uint32_t *spart) {
    using namespace gdma;
    static const hipError_t attr = [] {
        hipError_t e = allow_lds(gemm_bf16_kernel<OUT, false, EPI>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_kernel<OUT, true, EPI>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_split_kernel<false>, LDS_BYTES);
        if (e == hipSuccess) e = allow_lds(gemm_bf16_split_kernel<true>, LDS_BYTES);
        return e;
    }();
    if (attr != hipSuccess) return attr;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const dim3 block(256);
    const unsigned utm = (unsigned)tm, utn = (unsigned)tn;
    const bool tail = (2 * K) % BK != 0;
    const SplitPlan sp = plan_split(tm * tn, (int)((2 * K + BK - 1) / BK), spart != nullptr);
    if (sp.full > 0) {
        if (tail)
            hipLaunchKernelGGL((gemm_bf16_kernel<OUT, true, EPI>), dim3(sp.full), block, LDS_BYTES, s, x, w, M, N,
                               K, y, utm, utn, partial);
        else
            hipLaunchKernelGGL((gemm_bf16_kernel<OUT, false, EPI>), dim3(sp.full), block, LDS_BYTES, s, x, w, M, N,
                               K, y, utm, utn, partial);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (sp.splits > 1) {
        const dim3 grid(sp.tail * sp.splits);
        if (tail)
            hipLaunchKernelGGL(gemm_bf16_split_kernel<true>, grid, block, LDS_BYTES, s, x, w, M, N, K, utm, utn,
                               sp, spart, (EPI & kEpiAmax) ? partial : nullptr);
        else
            hipLaunchKernelGGL(gemm_bf16_split_kernel<false>, grid, block, LDS_BYTES, s, x, w, M, N, K, utm, utn,
                               sp, spart, (EPI & kEpiAmax) ? partial : nullptr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_fixup<OUT, EPI>(s, nullptr, nullptr, M, N, y, utm, utn, GROUP_M, partial, sp, spart);
    }
    return hipSuccess;
}

hipError_t launch_gemm_bf16(hipStream_t s, const uint16_t *x, const uint16_t *w, int64_t M,
                            int64_t N, int64_t K, int out_dtype, void *y, int epi, float *partial,
                            uint32_t *spart) {
    if (M == 0 || N == 0) return hipSuccess;
    if (out_dtype == 0 && epi == 0) return launch_bf16_paths<0, 0>(s, x, w, M, N, K, y, partial, spart);
    if (out_dtype != 1) return hipErrorInvalidValue;
    switch (epi) {
        case 0: return launch_bf16_paths<1, 0>(s, x, w, M, N, K, y, partial, spart);
        case 1: return launch_bf16_paths<1, 1>(s, x, w, M, N, K, y, partial, spart);
        case 2: return launch_bf16_paths<1, 2>(s, x, w, M, N, K, y, partial, spart);
        case 3: return launch_bf16_paths<1, 3>(s, x, w, M, N, K, y, partial, spart);
    }
    return hipErrorInvalidValue;
}

}  // namespace dmpq
