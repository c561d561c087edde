// gemm_int8.hip -- INT8 quantized linear Y = (A W^T) * sA[m] * sW[n] on
// gfx950 i8 MFMA.  Method: 6Bit-Diffusion routes volatile layers to INT8
// activations against INT8-converted weights (gist.science summaries §2.A).
//
// Both operands are K-contiguous, the natural MFMA layout: one lane's
// 16-byte LDS read is a 16-value k-slice of one A row (or W row).  The k
// order inside an MFMA does not matter for the result: A and W fragments use
// the same k mapping and int32 addition is exact.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid.  Workgroup tile 256 x 256,
// wave tile 128 x 128 = 4 x 4 MFMA 32x32x32 tiles (256 int32 accumulators per
// lane).  K advances 128 bytes per stage through a double-buffered LDS (rows
// padded to 144 bytes, conflict-free for the 32-row fragment reads); the
// next stage's global loads are in flight during the current stage's MFMAs,
// with one barrier per stage.
#include "device.hpp"
#include "gemm_common.hpp"
#include "internal.hpp"

namespace dmpq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace i8gemm {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int ROW = BK + 16;                  // padded LDS row, bytes
constexpr int STAGE = (BM + BN) * ROW;        // bytes per LDS stage
constexpr int LOADS = BM * BK / 16 / 256;     // 16-byte chunks per thread per operand
constexpr unsigned GROUP_M = 8;
}  // namespace i8gemm

template <int OUT>
__global__ __launch_bounds__(256, 1) void gemm_i8_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ W,
    const float *__restrict__ sw, int64_t M, int64_t N, int64_t K, void *__restrict__ y,
    unsigned tiles_m, unsigned tiles_n) {
    using namespace i8gemm;
    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const TileCoord tc = tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, GROUP_M);
    const int64_t m0 = (int64_t)tc.m * BM, n0 = (int64_t)tc.n * BN;

    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    // global -> register staging: chunk c = tid + 256*j covers row c/8, bytes (c%8)*16
    uint4 ra[LOADS], rw[LOADS];
    const int nk = (int)((K + BK - 1) / BK);

    // Out-of-range chunks (ragged M, N or K) load from a clamped in-range
    // address and are then replaced by zeros (a select on values, so no
    // pointer to a local zero is ever formed).
#define DMPQ_I8_GLOAD(k0)                                                                    \
    _Pragma("unroll") for (int j = 0; j < LOADS; j++) {                                      \
        const int c = tid + 256 * j;                                                         \
        const int r = c >> 3;                                                                \
        const int64_t gk = (k0) + (c & 7) * 16;                                              \
        const int64_t gm = m0 + r, gn = n0 + r;                                              \
        const int64_t gkc = gk < K ? gk : K - 16;                                            \
        const uint4 va = *reinterpret_cast<const uint4 *>(A + (gm < M ? gm : M - 1) * K + gkc); \
        const uint4 vw = *reinterpret_cast<const uint4 *>(W + (gn < N ? gn : N - 1) * K + gkc); \
        const bool oka = gm < M && gk < K, okw = gn < N && gk < K;                           \
        ra[j] = make_uint4(oka ? va.x : 0u, oka ? va.y : 0u, oka ? va.z : 0u, oka ? va.w : 0u); \
        rw[j] = make_uint4(okw ? vw.x : 0u, okw ? vw.y : 0u, okw ? vw.z : 0u, okw ? vw.w : 0u); \
    }
#define DMPQ_I8_SSTORE(buf)                                                                  \
    _Pragma("unroll") for (int j = 0; j < LOADS; j++) {                                      \
        const int c = tid + 256 * j;                                                         \
        const int r = c >> 3, kc = (c & 7) * 16;                                             \
        int8_t *base = lds + (buf) * STAGE;                                                  \
        *reinterpret_cast<uint4 *>(base + r * ROW + kc) = ra[j];                             \
        *reinterpret_cast<uint4 *>(base + (BM + r) * ROW + kc) = rw[j];                      \
    }

    DMPQ_I8_GLOAD(0)
    DMPQ_I8_SSTORE(0)
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
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            DMPQ_I8_SSTORE(cur ^ 1)
        }
        __syncthreads();
    }
#undef DMPQ_I8_GLOAD
#undef DMPQ_I8_SSTORE

    // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and rows
    // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
        if (col >= N) continue;
        const float swc = sw[col];
#pragma unroll
        for (int i = 0; i < 4; i++) {
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const int a = acc[i][j][r];
                const int64_t o = row * N + col;
                if constexpr (OUT == 2) {
                    static_cast<int32_t *>(y)[o] = a;
                } else {
                    const float v = ((float)a * sa[row]) * swc;
                    if constexpr (OUT == 0)
                        static_cast<float *>(y)[o] = v;
                    else
                        static_cast<uint16_t *>(y)[o] = (uint16_t)f32_to_bf16(v);
                }
            }
        }
    }
}

hipError_t launch_gemm_int8(hipStream_t s, const int8_t *qa, const float *sa, const int8_t *qw,
                            const float *sw, int64_t M, int64_t N, int64_t K, int out_dtype,
                            void *y) {
    using namespace i8gemm;
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tm * tn)), block(256);
    const size_t lds = 2 * STAGE;  // above the default dynamic-LDS limit: opt in once
    static const hipError_t attr = [] {
        const void *fns[3] = {reinterpret_cast<const void *>(gemm_i8_kernel<0>),
                              reinterpret_cast<const void *>(gemm_i8_kernel<1>),
                              reinterpret_cast<const void *>(gemm_i8_kernel<2>)};
        for (const void *f : fns) {
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(2 * STAGE));
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess) return attr;
    switch (out_dtype) {
        case 0:
            hipLaunchKernelGGL(gemm_i8_kernel<0>, grid, block, lds, s, qa, sa, qw, sw, M, N, K, y,
                               (unsigned)tm, (unsigned)tn);
            break;
        case 1:
            hipLaunchKernelGGL(gemm_i8_kernel<1>, grid, block, lds, s, qa, sa, qw, sw, M, N, K, y,
                               (unsigned)tm, (unsigned)tn);
            break;
        default:
            hipLaunchKernelGGL(gemm_i8_kernel<2>, grid, block, lds, s, qa, sa, qw, sw, M, N, K, y,
                               (unsigned)tm, (unsigned)tn);
            break;
    }
    return hipGetLastError();
}

}  // namespace dmpq
