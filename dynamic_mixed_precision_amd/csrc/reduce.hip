// reduce.hip -- Gamma predictor sums and the Temporal Delta Cache step.
// Method: 6Bit-Diffusion (gist.science summaries): Gamma is the relative L1
// distance between a block's output and input at the previous step (§2.A,
// "Mechanism"); TDC caches the residual delta out - in, compares the last two
// deltas, and either reuses the cached delta or recomputes (§2.B).
//
// All kernels stream bf16 in 16-byte vectors (8 elements).  Sums: each lane
// adds 8 non-negative fp32 terms (relative error <= 7 ulp of fp32, below
// 4.2e-7), then accumulates in fp64; workgroups reduce in a fixed tree and
// a second one-workgroup kernel adds the per-group partials in index order,
// so results are bit-identical from run to run (and no cross-workgroup fence
// is needed).
#include "device.hpp"
#include "internal.hpp"

namespace dmpq {

namespace {

__device__ __forceinline__ uint4 ld16(const uint16_t *p) {
    return load_nt16(p);
}

__device__ __forceinline__ void to8(const uint4 &a, float v[8]) {
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

// Reduce NS per-lane fp64 sums of one workgroup (fixed tree) and write them
// to partial[blockIdx.x * NS + j].  Must be called by every thread.
template <int NS>
__device__ void block_partials(double (&s)[NS], double *partial) {
    __shared__ double red[NS][4];
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < NS; j++) s[j] = wave_sum(s[j]);
    if ((tid & (kWave - 1)) == 0) {
#pragma unroll
        for (int j = 0; j < NS; j++) red[j][tid / kWave] = s[j];
    }
    __syncthreads();
    if (tid < NS)
        partial[(size_t)blockIdx.x * NS + tid] = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
}


}  // namespace

// Second stage of every sum: one workgroup adds the per-group partials in a
// fixed order (thread t takes partials t, t+256, ..., then a fixed tree), so
// the result does not depend on scheduling.  The loop has a fixed trip count
// (kIter >= nparts / 256) with guarded loads, so every load is issued before
// the first add waits: this kernel is pure latency, a few microseconds.
template <int NS, int kIter>
__global__ __launch_bounds__(256) void finalize_sums_kernel(const double *__restrict__ partial,
                                                            int nparts, double *__restrict__ out) {
    __shared__ double red[NS][4];
    const int tid = threadIdx.x;
    double v[kIter][NS];
#pragma unroll
    for (int k = 0; k < kIter; k++) {
        const int i = tid + 256 * k;
#pragma unroll
        for (int j = 0; j < NS; j++) v[k][j] = i < nparts ? partial[(size_t)i * NS + j] : 0.0;
    }
    double t[NS];
#pragma unroll
    for (int j = 0; j < NS; j++) {
        t[j] = 0.0;
#pragma unroll
        for (int k = 0; k < kIter; k++) t[j] += v[k][j];
    }
#pragma unroll
    for (int j = 0; j < NS; j++) t[j] = wave_sum(t[j]);
    if ((tid & (kWave - 1)) == 0) {
#pragma unroll
        for (int j = 0; j < NS; j++) red[j][tid / kWave] = t[j];
    }
    __syncthreads();
    if (tid < NS) out[tid] = (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
}

// Grids of the streaming kernels.  Each lane takes two 16-byte chunks per
// operand per iteration (chunks c and c + stride, all loads issued before
// any use), over few long-lived workgroups: 512 for Gamma, 256 (one per CU)
// for the TDC refresh and skip.  Same-box A/B against one chunk per lane
// over 1024 (Gamma, refresh) or up to 8192 (skip) workgroups, sums and
// outputs unchanged: refresh 71.5 against 76.9 us at 17776 x 3072 and 412
// against 486 us at 106306 x 3072; skip 54.3 against 54.7 and 316 against
// 392 us; Gamma 35.5 against 35.9 and 188 against 194 us.  Fewer
// workgroups also shrink the finalize work.
constexpr unsigned kGammaGroups = 512;
constexpr unsigned kTdcGroups = 256;
// The skip below 32 M chunks (256 M elements): one chunk per lane over up to
// 1024 workgroups, 2-4% faster there (17776 x 1920: 34.4 against 36.0 us;
// 17776 x 3072: 53.4 against 54.3 us), while two chunks over 256 win at the
// 1080p-like size (316 against 325 us).
constexpr int64_t kSkipLargeChunks = 32ll << 20;
constexpr unsigned kSkipSmallGroups = 1024;

// ---------------------------------------------------------------------------
// Gamma sums: S1 = sum |out - in|, S2 = sum |in|.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gamma_kernel(const uint16_t *__restrict__ xin,
                                                    const uint16_t *__restrict__ xout,
                                                    int64_t n, double *partial) {
    double s[2] = {0.0, 0.0};
    const int64_t nch = n / 8;
    const int64_t stride = (int64_t)gridDim.x * 256;
    auto add8 = [&](const uint4 &ra, const uint4 &rb) {
        float va[8], vb[8];
        to8(ra, va);
        to8(rb, vb);
        float f1 = 0.0f, f2 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
            f1 += __builtin_fabsf(vb[i] - va[i]);
            f2 += __builtin_fabsf(va[i]);
        }
        s[0] += (double)f1;
        s[1] += (double)f2;
    };
    int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; c + stride < nch; c += 2 * stride) {
        const uint4 a0 = ld16(xin + 8 * c), b0 = ld16(xout + 8 * c);
        const uint4 a1 = ld16(xin + 8 * (c + stride)), b1 = ld16(xout + 8 * (c + stride));
        add8(a0, b0);
        add8(a1, b1);
    }
    if (c < nch) add8(ld16(xin + 8 * c), ld16(xout + 8 * c));
    if (blockIdx.x == 0 && threadIdx.x < n - 8 * nch) {  // ragged tail, < 8 elements
        const int64_t i = 8 * nch + threadIdx.x;
        const float a = __uint_as_float((uint32_t)xin[i] << 16);
        const float b = __uint_as_float((uint32_t)xout[i] << 16);
        s[0] += (double)__builtin_fabsf(b - a);
        s[1] += (double)__builtin_fabsf(a);
    }
    block_partials<2>(s, partial);
}

hipError_t launch_gamma(hipStream_t st, const uint16_t *x_in, const uint16_t *x_out, int64_t n,
                        double *sums, const Workspace &ws) {
    const unsigned g = stride_grid(n / 8, 512, kGammaGroups);
    hipLaunchKernelGGL(gamma_kernel, dim3(g), dim3(256), 0, st, x_in, x_out, n, ws.partial);
    hipLaunchKernelGGL((finalize_sums_kernel<2, kGammaGroups / 256>), dim3(1), dim3(256), 0, st, ws.partial, (int)g,
                       sums);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// TDC skip: x_out = bf16(float(x_in) + float(delta)).
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(256) void tdc_skip_kernel(const uint16_t *__restrict__ xin,
                                                       const uint16_t *__restrict__ delta,
                                                       int64_t n, uint16_t *__restrict__ xout) {
    const int64_t nch = n / 8;
    const int64_t stride = (int64_t)gridDim.x * 256;
    auto skip8 = [&](int64_t ci, const uint4 &ra, const uint4 &rd) {
        float a[8], d[8];
        to8(ra, a);
        to8(rd, d);
        uint4 o;
        o.x = cvt_pk_bf16(a[0] + d[0], a[1] + d[1]);
        o.y = cvt_pk_bf16(a[2] + d[2], a[3] + d[3]);
        o.z = cvt_pk_bf16(a[4] + d[4], a[5] + d[5]);
        o.w = cvt_pk_bf16(a[6] + d[6], a[7] + d[7]);
        store_nt16(xout + 8 * ci, o);
    };
    int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if constexpr (U == 2) {
        for (; c + stride < nch; c += 2 * stride) {
            const uint4 a0 = ld16(xin + 8 * c), d0 = ld16(delta + 8 * c);
            const uint4 a1 = ld16(xin + 8 * (c + stride)), d1 = ld16(delta + 8 * (c + stride));
            skip8(c, a0, d0);
            skip8(c + stride, a1, d1);
        }
    }
    for (; c < nch; c += stride) skip8(c, ld16(xin + 8 * c), ld16(delta + 8 * c));
    if (blockIdx.x == 0 && threadIdx.x < n - 8 * nch) {
        const int64_t i = 8 * nch + threadIdx.x;
        const float a = __uint_as_float((uint32_t)xin[i] << 16);
        const float d = __uint_as_float((uint32_t)delta[i] << 16);
        xout[i] = (uint16_t)f32_to_bf16(a + d);
    }
}

hipError_t launch_tdc_skip(hipStream_t st, const uint16_t *x_in, const uint16_t *delta,
                           int64_t n, uint16_t *x_out) {
    if (n / 8 > kSkipLargeChunks) {
        const unsigned g = stride_grid(n / 8, 512, kTdcGroups);
        hipLaunchKernelGGL(tdc_skip_kernel<2>, dim3(g), dim3(256), 0, st, x_in, delta, n, x_out);
    } else {
        const unsigned g = stride_grid(n / 8, 256, kSkipSmallGroups);
        hipLaunchKernelGGL(tdc_skip_kernel<1>, dim3(g), dim3(256), 0, st, x_in, delta, n, x_out);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// TDC refresh: new = bf16(out - in); S1 = sum |out - in| (fp32 difference),
// S2 = sum |in|, S3 = sum |new - delta|, S4 = sum |delta| (only when a delta
// is cached), then delta <- new.
// ---------------------------------------------------------------------------
template <bool DV>
__device__ __forceinline__ void refresh8(const uint4 &ia, const uint4 &oa, const uint4 &da,
                                         double s[4], uint4 &nd) {
    float a[8], b[8], d[8];
    to8(ia, a);
    to8(oa, b);
    if (DV) to8(da, d);
    float f1 = 0.0f, f2 = 0.0f, f3 = 0.0f, f4 = 0.0f;
    float dn[8];
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 8; i++) dn[i] = b[i] - a[i];
#pragma unroll
    for (int i = 0; i < 4; i++) w[i] = cvt_pk_bf16(dn[2 * i], dn[2 * i + 1]);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        f1 += __builtin_fabsf(dn[i]);
        f2 += __builtin_fabsf(a[i]);
        if (DV) {
            const float nbf = (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
            f3 += __builtin_fabsf(nbf - d[i]);
            f4 += __builtin_fabsf(d[i]);
        }
    }
    nd = make_uint4(w[0], w[1], w[2], w[3]);
    s[0] += (double)f1;
    s[1] += (double)f2;
    if (DV) {
        s[2] += (double)f3;
        s[3] += (double)f4;
    }
}

template <bool DV>
__global__ __launch_bounds__(256) void tdc_refresh_kernel(const uint16_t *__restrict__ xin,
                                                          const uint16_t *__restrict__ xout,
                                                          uint16_t *__restrict__ delta,
                                                          int64_t n, double *partial) {
    double s[4] = {0.0, 0.0, 0.0, 0.0};
    const int64_t nch = n / 8;
    const int64_t stride = (int64_t)gridDim.x * 256;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; c + stride < nch; c += 2 * stride) {
        const int64_t c1 = c + stride;
        const uint4 i0 = ld16(xin + 8 * c), o0 = ld16(xout + 8 * c), d0 = DV ? ld16(delta + 8 * c) : zero;
        const uint4 i1 = ld16(xin + 8 * c1), o1 = ld16(xout + 8 * c1), d1 = DV ? ld16(delta + 8 * c1) : zero;
        uint4 nd0, nd1;
        refresh8<DV>(i0, o0, d0, s, nd0);
        store_nt16(delta + 8 * c, nd0);
        refresh8<DV>(i1, o1, d1, s, nd1);
        store_nt16(delta + 8 * c1, nd1);
    }
    if (c < nch) {
        uint4 nd;
        refresh8<DV>(ld16(xin + 8 * c), ld16(xout + 8 * c), DV ? ld16(delta + 8 * c) : zero, s, nd);
        store_nt16(delta + 8 * c, nd);
    }
    if (blockIdx.x == 0 && threadIdx.x < n - 8 * nch) {
        const int64_t i = 8 * nch + threadIdx.x;
        const float a = __uint_as_float((uint32_t)xin[i] << 16);
        const float b = __uint_as_float((uint32_t)xout[i] << 16);
        const float dn = b - a;
        const uint32_t nb = f32_to_bf16(dn);
        s[0] += (double)__builtin_fabsf(dn);
        s[1] += (double)__builtin_fabsf(a);
        if (DV) {
            const float d = __uint_as_float((uint32_t)delta[i] << 16);
            s[2] += (double)__builtin_fabsf(__uint_as_float(nb << 16) - d);
            s[3] += (double)__builtin_fabsf(d);
        }
        delta[i] = (uint16_t)nb;
    }
    block_partials<4>(s, partial);
}

hipError_t launch_tdc_refresh(hipStream_t st, const uint16_t *x_in, const uint16_t *x_out,
                              uint16_t *delta, int64_t n, int delta_valid, double *sums,
                              const Workspace &ws) {
    const unsigned g = stride_grid(n / 8, 512, kTdcGroups);
    if (delta_valid)
        hipLaunchKernelGGL(tdc_refresh_kernel<true>, dim3(g), dim3(256), 0, st, x_in, x_out,
                           delta, n, ws.partial);
    else
        hipLaunchKernelGGL(tdc_refresh_kernel<false>, dim3(g), dim3(256), 0, st, x_in, x_out,
                           delta, n, ws.partial);
    hipLaunchKernelGGL((finalize_sums_kernel<4, kTdcGroups / 256>), dim3(1), dim3(256), 0, st, ws.partial, (int)g,
                       sums);
    return hipGetLastError();
}

hipError_t launch_finalize_sums(hipStream_t st, const double *partial, int nparts, int ns,
                                double *out) {
    // up to kMaxSums * kMaxPartials / ns partials (the workspace's capacity)
    if (nparts < 0 || (int64_t)nparts * ns > (int64_t)kMaxSums * kMaxPartials) return hipErrorInvalidValue;
    switch (ns) {
        case 1:
            if (nparts <= 1024)
                hipLaunchKernelGGL((finalize_sums_kernel<1, 4>), dim3(1), dim3(256), 0, st, partial, nparts, out);
            else
                hipLaunchKernelGGL((finalize_sums_kernel<1, kMaxSums * kMaxPartials / 256>), dim3(1), dim3(256), 0,
                                   st, partial, nparts, out);
            break;
        case 2:
            hipLaunchKernelGGL((finalize_sums_kernel<2, kMaxSums * kMaxPartials / 512>), dim3(1), dim3(256), 0, st,
                               partial, nparts, out);
            break;
        case 4:
            hipLaunchKernelGGL((finalize_sums_kernel<4, kMaxPartials / 256>), dim3(1), dim3(256), 0, st, partial,
                               nparts, out);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dmpq
