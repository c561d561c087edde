// gemm_int8.hip -- INT8 quantized linear Y = (A W^T) * sA[m] * sW[n] on
// gfx950 i8 MFMA.  Method: 6Bit-Diffusion routes volatile layers to INT8
// activations against INT8-converted weights (gist.science summaries §2.A).
//
// Both operands are K-contiguous, the natural MFMA layout: one lane's
// 16-byte LDS read is one A row (or W row) slice of 16 k-values.  The MFMA's
// k order inside an instruction is irrelevant to the result because A and W
// fragments are loaded with the same k mapping and int32 addition is exact.
//
// Tiling: 256 threads = 4 waves in a 2 x 2 grid; workgroup tile 128 x 128,
// wave tile 64 x 64 = 2 x 2 MFMA 32x32x32 tiles; K staged through LDS 128
// bytes per row per step (rows padded by 16 bytes against bank conflicts),
// with the next tile prefetched into registers during the MFMAs.
#include "device.hpp"
#include "internal.hpp"

namespace dmpq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

namespace {
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int LDS_ROW = BK + 16;
constexpr int CHUNKS = BM * BK / 16 / 256;  // 16-byte chunks per thread per operand
}  // namespace

__global__ __launch_bounds__(256) void gemm_i8_kernel(const int8_t *__restrict__ A,
                                                      const float *__restrict__ sa,
                                                      const int8_t *__restrict__ W,
                                                      const float *__restrict__ sw, int64_t M,
                                                      int64_t N, int64_t K, int out_dtype,
                                                      void *__restrict__ y, unsigned tiles_n) {
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDS_ROW];
    __shared__ __attribute__((aligned(16))) int8_t Ws[BN * LDS_ROW];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * BM;
    const int64_t n0 = (int64_t)(blockIdx.x % tiles_n) * BN;

    v16i acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0;

    uint4 ra[CHUNKS], rw[CHUNKS];
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < CHUNKS; j++) {
            const int c = tid + 256 * j;
            const int r = c >> 3, kc = (c & 7) * 16;
            const int64_t gk = k0 + kc;
            const int64_t gm = m0 + r, gn = n0 + r;
            ra[j] = (gm < M && gk < K) ? *reinterpret_cast<const uint4 *>(A + gm * K + gk) : zero;
            rw[j] = (gn < N && gk < K) ? *reinterpret_cast<const uint4 *>(W + gn * K + gk) : zero;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int j = 0; j < CHUNKS; j++) {
            const int c = tid + 256 * j;
            const int r = c >> 3, kc = (c & 7) * 16;
            *reinterpret_cast<uint4 *>(As + r * LDS_ROW + kc) = ra[j];
            *reinterpret_cast<uint4 *>(Ws + r * LDS_ROW + kc) = rw[j];
        }
    };

    gload(0);
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (k0 + BK < K) gload(k0 + BK);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            v4i a[2], b[2];
            const int koff = ks + (lane >> 5) * 16;
#pragma unroll
            for (int i = 0; i < 2; i++) {
                a[i] = *reinterpret_cast<const v4i *>(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_ROW + koff);
                b[i] = *reinterpret_cast<const v4i *>(Ws + (wn * 64 + i * 32 + (lane & 31)) * LDS_ROW + koff);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }

    // Epilogue.  32x32 accumulator layout: lane l holds column l % 32 and rows
    // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
#pragma unroll
    for (int i = 0; i < 2; i++) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
            if (col >= N) continue;
            const float swc = sw[col];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= M) continue;
                const int a = acc[i][j][r];
                const int64_t o = row * N + col;
                if (out_dtype == 2) {
                    static_cast<int32_t *>(y)[o] = a;
                } else {
                    const float v = ((float)a * sa[row]) * swc;
                    if (out_dtype == 0)
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
    if (M == 0 || N == 0) return hipSuccess;
    const int64_t tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_i8_kernel, dim3((unsigned)(tm * tn)), dim3(256), 0, s, qa, sa, qw,
                       sw, M, N, K, out_dtype, y, (unsigned)tn);
    return hipGetLastError();
}

}  // namespace dmpq
