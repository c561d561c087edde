// quant.hip -- online block Hadamard fused with dynamic activation
// quantization (per-token INT8, two-level NVFP4), and the INT8 requant of an
// NVFP4 weight.  Method: 6Bit-Diffusion, DMPQ (gist.science summaries, §2.A:
// Hadamard on local activation blocks, then INT8 or NVFP4 by route; the
// Chinese summary's §2.A adds that weights are NVFP4 offline and converted
// when an INT8 GEMM needs them).
//
// Layout of the work: every lane owns whole 16-element blocks, so the
// Hadamard butterflies run entirely in registers with no lane exchange.  A
// block is 32 contiguous bytes of bf16; consecutive lanes own consecutive
// blocks, so a wave streams a contiguous 2 KB span per load pair.
#include "device.hpp"
#include "internal.hpp"

#include <float.h>

namespace dmpq {

// ---------------------------------------------------------------------------
// Row-wise INT8 quantization.  LPR lanes cooperate on one row; each lane holds
// BPL blocks (16*BPL fp32 values) in registers between the absmax reduction
// and the code write, so the row is read from memory exactly once.
// ---------------------------------------------------------------------------

// Source of a row's 16-blocks: bf16 activations, rotated unless flagged off.
struct Bf16Rows {
    const uint16_t *x;
    int flags;
    __device__ __forceinline__ void load(int64_t row, int64_t K, int b, float v[16]) const {
        const uint4 *p = reinterpret_cast<const uint4 *>(x + row * K + 16 * (int64_t)b);
        uint4 a0 = load_nt16(p);
        uint4 a1 = load_nt16(p + 1);
        unpack16(a0, a1, v);
        if (!(flags & 1)) fwht16(v);
    }
};

// Source of a row's 16-blocks: an NVFP4 weight dequantized to
// (E2M1 value * E4M3 value) * g in fp32 (nvfp4_block_values: the hardware
// E2M1 converter; the conversion is VALU-bound, and the bit decode it
// replaces cost about seven operations per element).
struct Nvfp4Rows {
    const uint8_t *codes;
    const uint8_t *scales;
    const float *g;
    __device__ __forceinline__ void load(int64_t row, int64_t K, int b, float v[16]) const {
        const uint2 c = *reinterpret_cast<const uint2 *>(codes + row * (K / 2) + 8 * (int64_t)b);
        nvfp4_block_values(c, e4m3_value(scales[row * (K / 16) + b]), *g, v);
    }
};

// One row group (256 / LPR rows) of the row quantizer; red: 4 floats of LDS.
// Every thread of the workgroup calls it with the same group.
template <int LPR, int BPL, class Src>
__device__ __forceinline__ void row_quant_int8_group(const Src &src, int64_t M, int64_t K,
                                                     int8_t *__restrict__ q, float *__restrict__ s_row,
                                                     int64_t group, float *red) {
    static_assert(LPR >= 16 && LPR <= 256 && 256 % LPR == 0, "lanes per row");
    constexpr int ROWS = 256 / LPR;
    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    const int64_t row = group * ROWS + tid / LPR;
    const int nblk = (int)(K / 16);
    const bool row_ok = row < M;

    float v[BPL][16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < BPL; i++) {
        const int b = lr + i * LPR;
        if (row_ok && b < nblk) {
            src.load(row, K, b, v[i]);
#pragma unroll
            for (int j = 0; j < 16; j++) amax = fmaxf(amax, __builtin_fabsf(v[i][j]));
        }
    }
    if constexpr (LPR <= kWave) {
        amax = group_max<LPR>(amax);
    } else {
        amax = wave_max(amax);
        if ((tid & (kWave - 1)) == 0) red[tid / kWave] = amax;
        __syncthreads();
        constexpr int WPR = LPR / kWave;
        const int w0 = (tid / LPR) * WPR;
        amax = red[w0];
#pragma unroll
        for (int w = 1; w < WPR; w++) amax = fmaxf(amax, red[w0 + w]);
    }
    if (!row_ok) return;

    // A row whose reciprocal 127/amax is not finite (amax zero, or below about
    // 3.7e-37) quantizes as a zero row: scale 0, codes 0.
    float inv = 127.0f / amax;
    const bool zero_row = !(inv <= FLT_MAX);
    if (zero_row) inv = 0.0f;
    if (lr == 0) s_row[row] = zero_row ? 0.0f : amax / 127.0f;
    int8_t *qr = q + row * K;
#pragma unroll
    for (int i = 0; i < BPL; i++) {
        const int b = lr + i * LPR;
        // a zero row stores zeros outright: its values may all be NaNs of any
        // payload (an NVFP4 weight with a NaN tensor scale)
        if (b < nblk)
            *reinterpret_cast<uint4 *>(qr + 16 * (int64_t)b) =
                zero_row ? make_uint4(0u, 0u, 0u, 0u) : int8_codes_magic(v[i], inv);
    }
}

template <int LPR, int BPL, class Src>
__global__ __launch_bounds__(256) void row_quant_int8_kernel(Src src, int64_t M, int64_t K,
                                                             int8_t *__restrict__ q,
                                                             float *__restrict__ s_row) {
    __shared__ float red[4];
    row_quant_int8_group<LPR, BPL>(src, M, K, q, s_row, blockIdx.x, red);
}

// The INT8 route's two row quantizations in one launch: workgroups
// 0 .. wgroups-1 convert the NVFP4 weight rows, the rest quantize the
// activation rows.  Both run the same row plan (they share K).  The weight
// rows go first: that conversion moves few bytes and is bound by latency,
// which the activation rows' stream then covers.
template <int LPR, int BPL>
__global__ __launch_bounds__(256) void row_quant_int8_w8_kernel(Nvfp4Rows wsrc, int64_t N,
                                                                int8_t *__restrict__ qw,
                                                                float *__restrict__ sw_row,
                                                                int64_t wgroups, Bf16Rows xsrc,
                                                                int64_t M, int8_t *__restrict__ q,
                                                                float *__restrict__ s_row, int64_t K) {
    __shared__ float red[4];
    if ((int64_t)blockIdx.x < wgroups)
        row_quant_int8_group<LPR, BPL>(wsrc, N, K, qw, sw_row, blockIdx.x, red);
    else
        row_quant_int8_group<LPR, BPL>(xsrc, M, K, q, s_row, blockIdx.x - wgroups, red);
}

// Pick lanes-per-row and blocks-per-lane for a row of nblk 16-blocks: the
// least idle lanes, then the fewest blocks per lane.  Fewer values held per
// lane means fewer registers, more waves in flight and more lanes loading:
// K = 3072 takes 64 lanes x 3 blocks rather than 32 x 6, K = 12288 takes
// 256 x 3 rather than 128 x 6.  Same-box timing of the INT8 quantizer at
// 17776 rows: 34.8 -> 32.3 us (K = 3072) and 111.8 -> 104.9 us (K = 12288).
struct RowPlan {
    int lpr, bpl;
};
static const int kBplChoices[] = {1, 2, 3, 4, 6, 8};

static bool plan_rows(int64_t K, RowPlan *out) {
    const int64_t nblk = K / 16;
    bool found = false;
    int64_t best_waste = 0;
    for (int lpr = 16; lpr <= 256; lpr *= 2) {
        for (int bpl : kBplChoices) {
            if ((int64_t)lpr * bpl < nblk) continue;
            const int64_t waste = (int64_t)lpr * bpl - nblk;
            // only the smallest bpl that covers the row for this lpr
            bool smaller_fits = false;
            for (int b2 : kBplChoices)
                if (b2 < bpl && (int64_t)lpr * b2 >= nblk) smaller_fits = true;
            if (smaller_fits) continue;
            if (!found || waste < best_waste || (waste == best_waste && bpl < out->bpl)) {
                found = true;
                best_waste = waste;
                out->lpr = lpr;
                out->bpl = bpl;
            }
        }
    }
    return found;
}

bool hq_int8_supported(int64_t K) {
    RowPlan p;
    return K > 0 && K % 16 == 0 && plan_rows(K, &p);
}

template <class Src, int LPR>
static hipError_t launch_rows_lpr(hipStream_t s, int bpl, const Src &src, int64_t M,
                                  int64_t K, int8_t *q, float *s_row) {
    const int64_t rows_per_group = 256 / LPR;
    const dim3 grid((unsigned)((M + rows_per_group - 1) / rows_per_group));
    switch (bpl) {
#define DMPQ_BPL(B)                                                                      \
    case B:                                                                              \
        hipLaunchKernelGGL((row_quant_int8_kernel<LPR, B, Src>), grid, dim3(256), 0, s, src, \
                           M, K, q, s_row);                                              \
        break;
        DMPQ_BPL(1) DMPQ_BPL(2) DMPQ_BPL(3) DMPQ_BPL(4) DMPQ_BPL(6) DMPQ_BPL(8)
#undef DMPQ_BPL
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class Src>
static hipError_t launch_rows(hipStream_t s, const Src &src, int64_t M, int64_t K, int8_t *q,
                              float *s_row) {
    RowPlan p;
    if (!plan_rows(K, &p)) return hipErrorInvalidValue;
    if (M == 0) return hipSuccess;
    switch (p.lpr) {
        case 16: return launch_rows_lpr<Src, 16>(s, p.bpl, src, M, K, q, s_row);
        case 32: return launch_rows_lpr<Src, 32>(s, p.bpl, src, M, K, q, s_row);
        case 64: return launch_rows_lpr<Src, 64>(s, p.bpl, src, M, K, q, s_row);
        case 128: return launch_rows_lpr<Src, 128>(s, p.bpl, src, M, K, q, s_row);
        case 256: return launch_rows_lpr<Src, 256>(s, p.bpl, src, M, K, q, s_row);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_hq_int8(hipStream_t s, const uint16_t *x, int64_t M, int64_t K, int flags,
                          int8_t *q, float *s_row) {
    return launch_rows(s, Bf16Rows{x, flags}, M, K, q, s_row);
}

// Per-row scales of the INT8 weight requantized from an NVFP4 weight, for the
// INT8 GEMM that converts the weight in its tile load: the same amax and
// reciprocal as row_quant_int8_kernel<..., Nvfp4Rows> (a maximum does not
// depend on the order), s = amax/127 and inv = 127/amax; a row whose
// reciprocal is not finite gets s = 0 and inv = 0 (the GEMM codes it as
// zeros).  One wave per row.
__global__ __launch_bounds__(256) void w8_row_scales_kernel(Nvfp4Rows src, int64_t N, int64_t K,
                                                            float *__restrict__ s_row,
                                                            float *__restrict__ inv_row) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N) return;  // the whole wave
    const int nblk = (int)(K / 16);
    float amax = 0.0f;
    for (int b = lane; b < nblk; b += kWave) {
        float v[16];
        src.load(row, K, b, v);
#pragma unroll
        for (int j = 0; j < 16; j++) amax = fmaxf(amax, __builtin_fabsf(v[j]));
    }
    amax = wave_max(amax);
    float inv = 127.0f / amax;
    const bool zero_row = !(inv <= FLT_MAX);
    if (zero_row) inv = 0.0f;
    if (lane == 0) {
        s_row[row] = zero_row ? 0.0f : amax / 127.0f;
        inv_row[row] = inv;
    }
}

hipError_t launch_w8_row_scales(hipStream_t s, const uint8_t *cw, const uint8_t *sw, const float *gw,
                                int64_t N, int64_t K, float *s_row, float *inv_row) {
    if (N == 0) return hipSuccess;
    hipLaunchKernelGGL(w8_row_scales_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s,
                       Nvfp4Rows{cw, sw, gw}, N, K, s_row, inv_row);
    return hipGetLastError();
}

hipError_t launch_w8_from_nvfp4(hipStream_t s, const uint8_t *cw, const uint8_t *sw,
                                const float *gw, int64_t N, int64_t K, int8_t *qw,
                                float *sw_row) {
    return launch_rows(s, Nvfp4Rows{cw, sw, gw}, N, K, qw, sw_row);
}

template <int LPR>
static hipError_t launch_w8_pair_lpr(hipStream_t s, int bpl, const Nvfp4Rows &w, int64_t N, int8_t *qw,
                                     float *sw_row, const Bf16Rows &x, int64_t M, int8_t *q,
                                     float *s_row, int64_t K) {
    const int64_t rows = 256 / LPR;
    const int64_t wg = (N + rows - 1) / rows, xg = (M + rows - 1) / rows;
    const dim3 grid((unsigned)(wg + xg));
    switch (bpl) {
#define DMPQ_BPL(B)                                                                            \
    case B:                                                                                    \
        hipLaunchKernelGGL((row_quant_int8_w8_kernel<LPR, B>), grid, dim3(256), 0, s, w, N, qw, \
                           sw_row, wg, x, M, q, s_row, K);                                     \
        break;
        DMPQ_BPL(1) DMPQ_BPL(2) DMPQ_BPL(3) DMPQ_BPL(4) DMPQ_BPL(6) DMPQ_BPL(8)
#undef DMPQ_BPL
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_hq_int8_w8(hipStream_t s, const uint16_t *x, int64_t M, int64_t K, int flags,
                             int8_t *q, float *s_row, const uint8_t *cw, const uint8_t *sw,
                             const float *gw, int64_t N, int8_t *qw, float *sw_row) {
    RowPlan p;
    if (!plan_rows(K, &p)) return hipErrorInvalidValue;
    if (M == 0 && N == 0) return hipSuccess;
    const Nvfp4Rows w{cw, sw, gw};
    const Bf16Rows xr{x, flags};
    switch (p.lpr) {
        case 16: return launch_w8_pair_lpr<16>(s, p.bpl, w, N, qw, sw_row, xr, M, q, s_row, K);
        case 32: return launch_w8_pair_lpr<32>(s, p.bpl, w, N, qw, sw_row, xr, M, q, s_row, K);
        case 64: return launch_w8_pair_lpr<64>(s, p.bpl, w, N, qw, sw_row, xr, M, q, s_row, K);
        case 128: return launch_w8_pair_lpr<128>(s, p.bpl, w, N, qw, sw_row, xr, M, q, s_row, K);
        case 256: return launch_w8_pair_lpr<256>(s, p.bpl, w, N, qw, sw_row, xr, M, q, s_row, K);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Outlier count of the Purified Delta Refresh check (gist.science summaries,
// §2.C: before a refresh writes the cached delta, a block input with a high
// outlier ratio is computed in full precision).  An element x of a token row
// (K channels, raw input, no Hadamard) counts when x^2 * K > kappa^2 * S with
// S = the row's sum of squares, all in fp64: each square of a bf16 value is
// exact, and S is added in a fixed order (per lane, then a fixed tree).
//
// The per-element test needs no fp64 work: x^2 * K is exact in fp64 (at most
// 16 + 15 significant bits) and increasing in |x|, so with R = kappa^2 * S
// the row's outliers are exactly the elements whose bf16 magnitude bits are
// at least b*, the least pattern b with v(b)^2 * K > R.  A square root gives
// a candidate c (the bf16 truncation of sqrt(R / K) through fp32); b* is c,
// c + 1 or c + 2 (the candidate's relative error, below 2^-23, is far under
// the bf16 spacing), decided by exact fp64 tests, once per row.  Elements then
// count by one integer compare.  A row whose R is not finite (an infinity or
// NaN in it) has no outliers, as in the fp64 test.  The row stays in
// registers (raw bf16 words) between the sum and the count.  Each workgroup
// writes its count to partial[blockIdx.x]; finalize_sums adds them.
// ---------------------------------------------------------------------------
template <int W>
__device__ __forceinline__ double group_sum_d(double v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, W);
    return v;
}

// bf16 magnitude pattern b (0 .. 0x7F80) as an fp64 value (exact)
__device__ __forceinline__ double bf16_mag(uint32_t b) { return (double)__uint_as_float(b << 16); }

// Least bf16 magnitude pattern b with v(b)^2 * K > R, for finite R >= 0
// (0x7F81, above every finite magnitude and infinity, when none qualifies).
__device__ __forceinline__ uint32_t outlier_threshold(double R, double dK) {
    const float tf = (float)__builtin_sqrt(R / dK);
    uint32_t c = __float_as_uint(tf) >> 16;  // truncation toward zero
    if (c > 0x7F80u) c = 0x7F80u;
#pragma unroll
    for (int d = 0; d < 3; d++) {  // b* is c, c + 1 or c + 2; c + 2 is tested too
        const uint32_t b = c + d;
        if (b <= 0x7F80u) {
            const double v = bf16_mag(b);
            if (v * v * dK > R) return b;
        }
    }
    return c + 3 <= 0x7F80u ? c + 3 : 0x7F81u;
}

template <int LPR, int BPL>
__global__ __launch_bounds__(256) void outlier_count_kernel(const uint16_t *__restrict__ x, int64_t M,
                                                           int64_t K, double kk,
                                                           double *__restrict__ partial) {
    static_assert(LPR >= 16 && LPR <= 256 && 256 % LPR == 0, "lanes per row");
    constexpr int ROWS = 256 / LPR;
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int lr = tid % LPR;
    const int nblk = (int)(K / 16);
    const double dK = (double)K;
    int cnt = 0;
    for (int64_t r0 = (int64_t)blockIdx.x * ROWS; r0 < M; r0 += (int64_t)gridDim.x * ROWS) {
        const int64_t row = r0 + tid / LPR;
        const bool row_ok = row < M;
        uint4 raw[BPL][2];
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < BPL; i++) {
            const int b = lr + i * LPR;
            if (row_ok && b < nblk) {
                const uint4 *p = reinterpret_cast<const uint4 *>(x + row * K + 16 * (int64_t)b);
                raw[i][0] = load_nt16(p);
                raw[i][1] = load_nt16(p + 1);
            } else {
                raw[i][0] = raw[i][1] = make_uint4(0u, 0u, 0u, 0u);
            }
            float v[16];
            unpack16(raw[i][0], raw[i][1], v);
            // one fused multiply-add: the square of a bf16 value is exact in
            // fp64, so fma(v, v, s) rounds exactly as s + v * v
#pragma unroll
            for (int j = 0; j < 16; j++) s = __builtin_fma((double)v[j], (double)v[j], s);
        }
        if constexpr (LPR <= kWave) {
            s = group_sum_d<LPR>(s);
        } else {
            s = wave_sum(s);
            if ((tid & (kWave - 1)) == 0) red[tid / kWave] = s;
            __syncthreads();
            constexpr int WPR = LPR / kWave;
            const int w0 = (tid / LPR) * WPR;
            double t = red[w0];
#pragma unroll
            for (int w = 1; w < WPR; w++) t += red[w0 + w];
            s = t;
            __syncthreads();
        }
        const double R = kk * s;
        // a non-finite R (or a row past M) counts nothing: 0xFFFF is above
        // every magnitude; zero padding never counts either (threshold >= 1)
        const uint32_t thr = (row_ok && R <= 1.7976931348623157e308) ? outlier_threshold(R, dK) : 0xFFFFu;
        // the wave's count per element slot: a ballot of the compare and a
        // scalar population count, so the sum across lanes is free
#pragma unroll
        for (int i = 0; i < BPL; i++) {
            const uint32_t w[8] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w,
                                   raw[i][1].x, raw[i][1].y, raw[i][1].z, raw[i][1].w};
#pragma unroll
            for (int j = 0; j < 8; j++) {
                cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64((w[j] & 0x7FFFu) >= thr));
                cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(((w[j] >> 16) & 0x7FFFu) >= thr));
            }
        }
    }
    // cnt is the wave's count (the same in every lane)
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = (double)cnt;
    __syncthreads();
    if (tid == 0) partial[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// One count per workgroup: the workspace holds kMaxSums * kMaxPartials of
// them, so every row group of a 17776-token input gets its own workgroup.
constexpr int kOutlierGroups = kMaxSums * kMaxPartials;

hipError_t launch_outlier_count(hipStream_t s, const uint16_t *x, int64_t M, int64_t K,
                                double kappa, double *count, const Workspace &ws) {
    RowPlan p;
    if (!plan_rows(K, &p)) return hipErrorInvalidValue;
    const double kk = kappa * kappa;
    const int64_t rows = 256 / p.lpr;
    const int64_t groups64 = (M + rows - 1) / rows;
    const int groups = (int)(groups64 < kOutlierGroups ? groups64 : kOutlierGroups);
    if (groups > 0) {
        const dim3 grid((unsigned)groups);
        switch (p.lpr * 16 + p.bpl) {
#define DMPQ_OC(L, B)                                                                            \
    case L * 16 + B:                                                                             \
        hipLaunchKernelGGL((outlier_count_kernel<L, B>), grid, dim3(256), 0, s, x, M, K, kk, ws.partial); \
        break;
#define DMPQ_OC_L(L) DMPQ_OC(L, 1) DMPQ_OC(L, 2) DMPQ_OC(L, 3) DMPQ_OC(L, 4) DMPQ_OC(L, 6) DMPQ_OC(L, 8)
            DMPQ_OC_L(16) DMPQ_OC_L(32) DMPQ_OC_L(64) DMPQ_OC_L(128) DMPQ_OC_L(256)
#undef DMPQ_OC_L
#undef DMPQ_OC
            default: return hipErrorInvalidValue;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_finalize_sums(s, ws.partial, groups, 1, count);
}

// ---------------------------------------------------------------------------
// NVFP4, pass 1: absmax of the rotated tensor.  Each workgroup writes the max
// of its share to partial[blockIdx.x]; pass 2 reduces the partials itself
// (max is order independent).  No cross-workgroup fence is needed: the kernel
// boundary orders the two passes.  At most 512 workgroups: every pass-2
// workgroup first reads all the partials, and a same-box A/B (codes
// identical) put 512 ahead of 1024 by 2.5-5% with the input in cache (47.0
// against 48.2 us at 17776 x 3072, 173 against 179 us at x 12288) and 1-3%
// cold; 256, 384 and 768 were between or behind.
// ---------------------------------------------------------------------------
constexpr int kAmaxGroups = 512;

__global__ __launch_bounds__(256) void nvfp4_amax_kernel(const uint16_t *__restrict__ x,
                                                         int64_t nblocks, int flags,
                                                         float *__restrict__ partial) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    float m = 0.0f;
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t b = (int64_t)blockIdx.x * 256 + tid;
    for (; b + stride < nblocks; b += 2 * stride) {  // two blocks in flight per lane
        const uint4 *p0 = reinterpret_cast<const uint4 *>(x + 16 * b);
        const uint4 *p1 = reinterpret_cast<const uint4 *>(x + 16 * (b + stride));
        uint4 a0 = p0[0], a1 = p0[1];
        uint4 c0 = p1[0], c1 = p1[1];
        float v[16], w[16];
        unpack16(a0, a1, v);
        unpack16(c0, c1, w);
        if (!(flags & 1)) {
            fwht16(v);
            fwht16(w);
        }
#pragma unroll
        for (int j = 0; j < 16; j++) m = fmaxf(m, fmaxf(__builtin_fabsf(v[j]), __builtin_fabsf(w[j])));
    }
    if (b < nblocks) {
        const uint4 *p0 = reinterpret_cast<const uint4 *>(x + 16 * b);
        float v[16];
        unpack16(p0[0], p0[1], v);
        if (!(flags & 1)) fwht16(v);
#pragma unroll
        for (int j = 0; j < 16; j++) m = fmaxf(m, __builtin_fabsf(v[j]));
    }
    m = wave_max(m);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
    __syncthreads();
    if (tid == 0) partial[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------------------
// NVFP4, pass 2: reduce the pass-1 partials to the tensor amax A, then per
// 16-block the E4M3 scale and the E2M1 codes.  The flat block index b
// addresses codes (8 bytes per block) and scales (1 byte per block) directly
// because K is a multiple of 16.  Codes use the gfx950 converter
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 (round to nearest even,
// saturating at 6, sign kept), which matches the E2M1 rule for every finite
// fp32 input.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e2m1x8(const float *y) {
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
    return w;
}

__global__ __launch_bounds__(256) void nvfp4_quant_kernel(const uint16_t *__restrict__ x,
                                                          int64_t nblocks, int flags,
                                                          const float *__restrict__ partial,
                                                          int nparts, uint8_t *__restrict__ codes,
                                                          uint8_t *__restrict__ scales,
                                                          float *__restrict__ g_out) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    float a = 0.0f;
    for (int i = tid; i < nparts; i += 256) a = fmaxf(a, partial[i]);
    a = wave_max(a);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = a;
    __syncthreads();
    const float A = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float g = A / 2688.0f;
    if (blockIdx.x == 0 && tid == 0) *g_out = g;

    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t b = (int64_t)blockIdx.x * 256 + tid; b < nblocks; b += stride) {
        const uint4 *p = reinterpret_cast<const uint4 *>(x + 16 * b);
        uint4 a0 = load_nt16(p);
        uint4 a1 = load_nt16(p + 1);
        float v[16];
        unpack16(a0, a1, v);
        if (!(flags & 1)) {
            fwht16(v);
        } else {
            // NaN codes +0, but the hardware converter saturates it to +-6 by
            // sign.  A rotated block needs no care: every rotated value sums
            // all 16 inputs, so a NaN makes the whole block NaN, its amax 0
            // and its codes the zero-scale zeros.  Unrotated (a test hook),
            // a NaN sits among finite values and is replaced by +0 here
            // (the amax ignores NaNs either way).
#pragma unroll
            for (int j = 0; j < 16; j++) v[j] = (v[j] == v[j]) ? v[j] : 0.0f;
        }
        float ab = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; j++) ab = fmaxf(ab, __builtin_fabsf(v[j]));
        uint32_t e = 0u;
        float S = 0.0f;
        if (A > 0.0f) {
            const float r = ab / A;
            e = e4m3_encode_nonneg(r * 448.0f);
            S = e4m3_value(e) * g;
        }
        uint32_t w0 = 0u, w1 = 0u;
        if (S >= FLT_MIN) {
            const float inv = 1.0f / S;
#pragma unroll
            for (int j = 0; j < 16; j++) v[j] = v[j] * inv;
            w0 = e2m1x8(v);
            w1 = e2m1x8(v + 8);
        }
        *reinterpret_cast<uint2 *>(codes + 8 * b) = make_uint2(w0, w1);
        scales[b] = (uint8_t)e;
    }
}

// DMPQ_AMAX_GIVEN: one workgroup folds the producer GEMM's per-tile maxima
// into partial[0] (every read precedes the barrier, so the in-place write is
// safe), and pass 2 then reduces that single partial.
__global__ __launch_bounds__(1024) void amax_fold_kernel(float *__restrict__ partial, int64_t n) {
    __shared__ float red[16];
    const int tid = threadIdx.x;
    float m = 0.0f;
    for (int64_t i = tid; i < n; i += 1024) m = fmaxf(m, partial[i]);
    m = wave_max(m);
    if ((tid & (kWave - 1)) == 0) red[tid / kWave] = m;
    __syncthreads();
    if (tid == 0) {
        float a = red[0];
        for (int w = 1; w < 16; w++) a = fmaxf(a, red[w]);
        partial[0] = a;
    }
}

int64_t hq_nvfp4_partials(int64_t M, int64_t K) {
    return stride_grid(M * (K / 16), 256 * 4, kAmaxGroups);
}

hipError_t launch_hq_nvfp4(hipStream_t s, const uint16_t *x, int64_t M, int64_t K, int flags,
                           uint8_t *codes, uint8_t *scales, float *g, const Workspace &ws) {
    const int64_t nblocks = M * (K / 16);
    float *partial = reinterpret_cast<float *>(ws.partial);
    unsigned nparts;
    if (flags & 2) {
        hipLaunchKernelGGL(amax_fold_kernel, dim3(1), dim3(1024), 0, s, partial, gemm_tiles(M, K));
        nparts = 1;
    } else {
        nparts = (unsigned)hq_nvfp4_partials(M, K);
        hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(nparts), dim3(256), 0, s, x, nblocks, flags, partial);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned gb = stride_grid(nblocks, 256 * 2, 8192);
    hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(gb), dim3(256), 0, s, x, nblocks, flags & 1, partial,
                       (int)nparts, codes, scales, g);
    return hipGetLastError();
}

}  // namespace dmpq
