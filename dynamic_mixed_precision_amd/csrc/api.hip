// api.hip -- the C ABI of libdmpq (declared in include/dmpq.h): argument
// validation, per-thread error messages, the host-side router and TDC
// bookkeeping, and dispatch to the gfx950 kernels.
#include "dmpq.h"
#include "internal.hpp"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

using namespace dmpq;

namespace {

thread_local char g_err[512] = "";

dmpq_status fail(dmpq_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

dmpq_status ok() {
    g_err[0] = '\0';
    return DMPQ_OK;
}

dmpq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(DMPQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A device pointer must be non-NULL and 16-byte aligned, except that a buffer
// of zero elements may be NULL (torch hands out NULL for empty tensors).
#define REQUIRE_PTR_NF(fn, p, count)                                                     \
    do {                                                                                 \
        if ((count) > 0 && !(p))                                                         \
            return fail(DMPQ_ERR_INVALID_ARG, "%s: %s is NULL", (fn), #p);               \
        if ((p) && !aligned16(p))                                                        \
            return fail(DMPQ_ERR_MISALIGNED, "%s: %s is not 16-byte aligned", (fn), #p); \
    } while (0)
#define REQUIRE_PTR_N(p, count) REQUIRE_PTR_NF(__func__, p, count)
#define REQUIRE_PTR(p) REQUIRE_PTR_N(p, 1)

#define REQUIRE_HOST(p)                                                                 \
    do {                                                                                \
        if (!(p)) return fail(DMPQ_ERR_INVALID_ARG, "%s: %s is NULL", __func__, #p);    \
    } while (0)

dmpq_status check_k(const char *fn, int64_t K) {
    if (K <= 0 || K % 16 != 0)
        return fail(DMPQ_ERR_BAD_SHAPE, "%s: K = %lld must be a positive multiple of 16", fn,
                    (long long)K);
    return DMPQ_OK;
}

dmpq_status check_ws(const char *fn, const void *ws, size_t bytes) {
    if (!ws) return fail(DMPQ_ERR_WORKSPACE, "%s: workspace is NULL", fn);
    if (!aligned16(ws)) return fail(DMPQ_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (bytes < kWsBytes)
        return fail(DMPQ_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, bytes,
                    kWsBytes);
    return DMPQ_OK;
}

// Workspace of a *_ex GEMM: the fused-amax maxima (one float per 256 x 256
// tile, rounded up to 256 bytes), then the split area.
size_t gemm_slot_bytes(int64_t M, int64_t N) {
    return ((size_t)gemm_tiles(M, N) * sizeof(float) + 255) / 256 * 256;
}

// Epilogue of a *_ex GEMM: known bits, bf16 output for a nonzero epilogue,
// and for the fused amax N % 16 == 0 and a workspace that holds one float per
// tile.  `outs`: the output types the GEMM itself accepts.
dmpq_status check_epilogue(const char *fn, int64_t M, int64_t N, int out_dtype, int outs,
                           int epilogue, const void *ws, size_t ws_bytes) {
    if (epilogue & ~(DMPQ_EPI_GELU | DMPQ_EPI_NVFP4_AMAX))
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown epilogue %d", fn, epilogue);
    if (out_dtype < 0 || out_dtype > 2 || !((outs >> out_dtype) & 1))
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown out_dtype %d", fn, out_dtype);
    if (epilogue != 0 && out_dtype != DMPQ_OUT_BF16)
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: epilogues need DMPQ_OUT_BF16 (got %d)", fn, out_dtype);
    if (ws && !aligned16(ws)) return fail(DMPQ_ERR_MISALIGNED, "%s: workspace is not 16-byte aligned", fn);
    if (epilogue & DMPQ_EPI_NVFP4_AMAX) {
        if (N % 16 != 0)
            return fail(DMPQ_ERR_BAD_SHAPE, "%s: the fused amax needs N %% 16 == 0 (N = %lld)", fn,
                        (long long)N);
        const size_t need = (size_t)gemm_tiles(M, N) * sizeof(float);
        if (!ws) return fail(DMPQ_ERR_WORKSPACE, "%s: workspace is NULL", fn);
        if (ws_bytes < need)
            return fail(DMPQ_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, ws_bytes, need);
    }
    return DMPQ_OK;
}

// The split area of a *_ex GEMM's workspace, or NULL when it is too small.
uint32_t *split_area(void *ws, size_t ws_bytes, int64_t M, int64_t N) {
    const size_t off = gemm_slot_bytes(M, N);
    if (!ws || ws_bytes < off + kSplitAreaBytes) return nullptr;
    return reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(ws) + off);
}

double rel_ratio(double num, double den) {
    if (den == 0.0) return num == 0.0 ? 0.0 : INFINITY;
    return num / den;
}

}  // namespace

namespace dmpq {
// For entry points defined in other translation units.
dmpq_status set_last_error(dmpq_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

// The arguments of the NVFP4 quantizer other than its workspace, checked
// in the name of entry point fn (also before the no-workspace entry point
// makes any HIP call).
dmpq_status check_hq_nvfp4_args(const char *fn, const uint16_t *x, int64_t M, int64_t K, int flags,
                                const uint8_t *codes, const uint8_t *scales, const float *d_g) {
    if (M < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: M = %lld < 0", fn, (long long)M);
    if (dmpq_status s = check_k(fn, K)) return s;
    REQUIRE_PTR_NF(fn, x, M);
    REQUIRE_PTR_NF(fn, codes, M);
    REQUIRE_PTR_NF(fn, scales, M);
    REQUIRE_PTR_NF(fn, d_g, 1);
    if (flags & ~(DMPQ_NO_HADAMARD | DMPQ_AMAX_GIVEN))
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown flags %d", fn, flags);
    if ((flags & DMPQ_NO_HADAMARD) && (flags & DMPQ_AMAX_GIVEN))
        return fail(DMPQ_ERR_INVALID_ARG, "%s: DMPQ_AMAX_GIVEN needs the rotation", fn);
    return DMPQ_OK;
}
}  // namespace dmpq

extern "C" {

const char *dmpq_last_error(void) { return g_err; }

const char *dmpq_version(void) { return "dmpq 0.1 gfx950"; }

size_t dmpq_workspace_bytes(int op, int64_t M, int64_t K) {
    switch (op) {
        case DMPQ_OP_GEMM_AMAX: {
            if (M < 0 || K < 0) return 0;
            const size_t tiles = (size_t)gemm_tiles(M, K);
            return tiles * sizeof(float) > kWsBytes ? tiles * sizeof(float) : kWsBytes;
        }
        case DMPQ_OP_GEMM:
            if (M < 0 || K < 0) return 0;
            return gemm_slot_bytes(M, K) + kSplitAreaBytes;
        case DMPQ_OP_GEMM_W4:  // the fused-amax slots, then s_row and inv_row of the weight
            if (M < 0 || K < 0) return 0;
            return gemm_slot_bytes(M, K) + 2 * sizeof(float) * (size_t)K;
        case DMPQ_OP_GAMMA:
        case DMPQ_OP_QUANT_NVFP4:
        case DMPQ_OP_TDC:
        case DMPQ_OP_PREP_WEIGHT:
        case DMPQ_OP_OUTLIER: return kWsBytes;
    }
    return 0;
}

dmpq_status dmpq_gamma_sums(hipStream_t stream, const uint16_t *x_in, const uint16_t *x_out,
                            int64_t n, double *d_sums2, void *ws, size_t ws_bytes) {
    if (n < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: n = %lld < 0", __func__, (long long)n);
    REQUIRE_PTR_N(x_in, n);
    REQUIRE_PTR_N(x_out, n);
    REQUIRE_PTR(d_sums2);
    if (dmpq_status s = check_ws(__func__, ws, ws_bytes)) return s;
    return hip_status(launch_gamma(stream, x_in, x_out, n, d_sums2, Workspace(ws)), __func__);
}

dmpq_status dmpq_gate_and_route(const double *h_sums2, int n_lin, const double *h_alpha,
                                const double *h_beta, double tau, double *h_gamma_out,
                                double *h_err_out, uint8_t *h_route_out) {
    if (n_lin < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: n_lin = %d < 0", __func__, n_lin);
    REQUIRE_HOST(h_route_out);
    if (!h_sums2) {  // Gamma missing: INT8 for every linear
        if (h_gamma_out) *h_gamma_out = NAN;
        for (int l = 0; l < n_lin; l++) {
            if (h_err_out) h_err_out[l] = NAN;
            h_route_out[l] = DMPQ_ROUTE_INT8;
        }
        return ok();
    }
    REQUIRE_HOST(h_alpha);
    REQUIRE_HOST(h_beta);
    const double gamma = rel_ratio(h_sums2[0], h_sums2[1]);
    if (h_gamma_out) *h_gamma_out = gamma;
    for (int l = 0; l < n_lin; l++) {
        const double e = h_alpha[l] * gamma + h_beta[l];
        if (h_err_out) h_err_out[l] = e;
        h_route_out[l] = e > tau ? DMPQ_ROUTE_INT8 : DMPQ_ROUTE_NVFP4;
    }
    return ok();
}

dmpq_status dmpq_hadamard_quant_int8(hipStream_t stream, const uint16_t *x, int64_t M,
                                     int64_t K, int flags, int8_t *q, float *s_row) {
    if (M < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: M = %lld < 0", __func__, (long long)M);
    if (dmpq_status s = check_k(__func__, K)) return s;
    REQUIRE_PTR_N(x, M);
    REQUIRE_PTR_N(q, M);
    REQUIRE_PTR_N(s_row, M);
    if (flags & ~DMPQ_NO_HADAMARD) return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown flags %d", __func__, flags);
    if (!hq_int8_supported(K))
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld exceeds 32768", __func__, (long long)K);
    return hip_status(launch_hq_int8(stream, x, M, K, flags, q, s_row), __func__);
}

dmpq_status dmpq_hadamard_quant_nvfp4(hipStream_t stream, const uint16_t *x, int64_t M,
                                      int64_t K, int flags, uint8_t *codes, uint8_t *scales,
                                      float *d_g, void *ws, size_t ws_bytes) {
    if (dmpq_status s = check_hq_nvfp4_args(__func__, x, M, K, flags, codes, scales, d_g)) return s;
    if (dmpq_status s = check_ws(__func__, ws, ws_bytes)) return s;
    if ((flags & DMPQ_AMAX_GIVEN) && ws_bytes < dmpq_workspace_bytes(DMPQ_OP_GEMM_AMAX, M, K))
        return fail(DMPQ_ERR_WORKSPACE, "%s: workspace has %zu bytes, the producer's tile maxima need %zu",
                    __func__, ws_bytes, dmpq_workspace_bytes(DMPQ_OP_GEMM_AMAX, M, K));
    return hip_status(launch_hq_nvfp4(stream, x, M, K, flags, codes, scales, d_g, Workspace(ws)),
                      __func__);
}

static dmpq_status check_gemm(const char *fn, int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0)
        return fail(DMPQ_ERR_BAD_SHAPE, "%s: M = %lld, N = %lld must be >= 0", fn, (long long)M,
                    (long long)N);
    if (M > (int64_t)INT32_MAX * 128 || N > (int64_t)INT32_MAX)
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: M or N too large", fn);
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (tiles > (int64_t)UINT32_MAX) return fail(DMPQ_ERR_UNSUPPORTED, "%s: too many tiles", fn);
    if (K > kMaxGemmK)
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld exceeds %lld", fn, (long long)K, (long long)kMaxGemmK);
    return check_k(fn, K);
}

dmpq_status dmpq_qgemm_int8(hipStream_t stream, const int8_t *qa, const float *sa,
                            const int8_t *qw, const float *sw, int64_t M, int64_t N, int64_t K,
                            int out_dtype, void *y) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    REQUIRE_PTR_N(qa, M);
    REQUIRE_PTR_N(sa, M);
    REQUIRE_PTR_N(qw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR_N(y, M * N);
    if (out_dtype != DMPQ_OUT_F32 && out_dtype != DMPQ_OUT_BF16 && out_dtype != DMPQ_OUT_I32)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown out_dtype %d", __func__, out_dtype);
    return hip_status(launch_gemm_int8(stream, qa, sa, qw, sw, M, N, K, out_dtype, y, 0, nullptr, nullptr),
                      __func__);
}

dmpq_status dmpq_qgemm_int8_ex(hipStream_t stream, const int8_t *qa, const float *sa,
                               const int8_t *qw, const float *sw, int64_t M, int64_t N, int64_t K,
                               int out_dtype, void *y, int epilogue, void *ws, size_t ws_bytes) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    REQUIRE_PTR_N(qa, M);
    REQUIRE_PTR_N(sa, M);
    REQUIRE_PTR_N(qw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR_N(y, M * N);
    if (dmpq_status s = check_epilogue(__func__, M, N, out_dtype, 7, epilogue, ws, ws_bytes)) return s;
    return hip_status(launch_gemm_int8(stream, qa, sa, qw, sw, M, N, K, out_dtype, y, epilogue,
                                       static_cast<float *>(ws), split_area(ws, ws_bytes, M, N)),
                      __func__);
}

dmpq_status dmpq_qgemm_int8_from_nvfp4(hipStream_t stream, const int8_t *qa, const float *sa,
                                       const uint8_t *cw, const uint8_t *sw, const float *d_gw,
                                       int64_t M, int64_t N, int64_t K, int out_dtype, void *y,
                                       int epilogue, void *ws, size_t ws_bytes) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    if (K % 128 != 0)
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld is not a multiple of 128", __func__, (long long)K);
    REQUIRE_PTR_N(qa, M);
    REQUIRE_PTR_N(sa, M);
    REQUIRE_PTR_N(cw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR(d_gw);
    REQUIRE_PTR_N(y, M * N);
    if (dmpq_status s = check_epilogue(__func__, M, N, out_dtype, 7, epilogue, ws, ws_bytes)) return s;
    const size_t need = dmpq_workspace_bytes(DMPQ_OP_GEMM_W4, M, N);
    if (!ws) return fail(DMPQ_ERR_WORKSPACE, "%s: workspace is NULL", __func__);
    if (ws_bytes < need)
        return fail(DMPQ_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", __func__, ws_bytes, need);
    if (M == 0 || N == 0) return ok();
    float *s_row = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + gemm_slot_bytes(M, N));
    float *inv_row = s_row + N;
    hipError_t e = launch_w8_row_scales(stream, cw, sw, d_gw, N, K, s_row, inv_row);
    if (e == hipSuccess)
        e = launch_gemm_int8_w4(stream, qa, sa, cw, sw, d_gw, s_row, inv_row, M, N, K, out_dtype, y, epilogue,
                                static_cast<float *>(ws));
    return hip_status(e, __func__);
}

dmpq_status dmpq_qgemm_nvfp4(hipStream_t stream, const uint8_t *ca, const uint8_t *sa,
                             const float *d_ga, const uint8_t *cw, const uint8_t *sw,
                             const float *d_gw, int64_t M, int64_t N, int64_t K, int out_dtype,
                             void *y, int variant) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    if (variant == DMPQ_FP4_SCALED_MFMA && ((M + 127) / 128) * ((N + 127) / 128) > (int64_t)UINT32_MAX)
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: too many tiles", __func__);
    REQUIRE_PTR_N(ca, M);
    REQUIRE_PTR_N(sa, M);
    REQUIRE_PTR_N(d_ga, M * N);
    REQUIRE_PTR_N(cw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR_N(d_gw, M * N);
    REQUIRE_PTR_N(y, M * N);
    if (out_dtype != DMPQ_OUT_F32 && out_dtype != DMPQ_OUT_BF16)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown out_dtype %d", __func__, out_dtype);
    if (variant != DMPQ_FP4_BF16_DEQUANT && variant != DMPQ_FP4_SCALED_MFMA)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown variant %d", __func__, variant);
    return hip_status(launch_gemm_nvfp4(stream, ca, sa, d_ga, cw, sw, d_gw, M, N, K, out_dtype,
                                        y, variant, 0, nullptr, nullptr),
                      __func__);
}

dmpq_status dmpq_qgemm_nvfp4_ex(hipStream_t stream, const uint8_t *ca, const uint8_t *sa,
                                const float *d_ga, const uint8_t *cw, const uint8_t *sw,
                                const float *d_gw, int64_t M, int64_t N, int64_t K,
                                int out_dtype, void *y, int epilogue, void *ws, size_t ws_bytes) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    REQUIRE_PTR_N(ca, M);
    REQUIRE_PTR_N(sa, M);
    REQUIRE_PTR_N(d_ga, M * N);
    REQUIRE_PTR_N(cw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR_N(d_gw, M * N);
    REQUIRE_PTR_N(y, M * N);
    if (dmpq_status s = check_epilogue(__func__, M, N, out_dtype, 3, epilogue, ws, ws_bytes)) return s;
    return hip_status(launch_gemm_nvfp4(stream, ca, sa, d_ga, cw, sw, d_gw, M, N, K, out_dtype, y,
                                        DMPQ_FP4_BF16_DEQUANT, epilogue, static_cast<float *>(ws),
                                        split_area(ws, ws_bytes, M, N)),
                      __func__);
}

dmpq_status dmpq_tdc_init(dmpq_tdc_state *h_st) {
    REQUIRE_HOST(h_st);
    memset(h_st, 0, sizeof *h_st);
    h_st->d = INFINITY;
    h_st->gamma = NAN;
    return ok();
}

dmpq_status dmpq_tdc_decide(const dmpq_tdc_state *h_st, const dmpq_tdc_params *h_p,
                            int *h_skip) {
    REQUIRE_HOST(h_st);
    REQUIRE_HOST(h_p);
    REQUIRE_HOST(h_skip);
    *h_skip = h_st->n_refresh >= 2 && h_st->delta_valid && h_st->d < h_p->eps_sim &&
              h_st->acc + h_st->d <= h_p->delta_acc;
    return ok();
}

dmpq_status dmpq_tdc_step(hipStream_t stream, int mode, const uint16_t *x_in, uint16_t *x_out,
                          uint16_t *delta, int64_t n, int delta_valid, double *d_sums4,
                          void *ws, size_t ws_bytes) {
    if (n < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: n = %lld < 0", __func__, (long long)n);
    REQUIRE_PTR_N(x_in, n);
    REQUIRE_PTR_N(x_out, n);
    REQUIRE_PTR_N(delta, n);
    if (mode == DMPQ_TDC_SKIP) {
        if (!delta_valid)
            return fail(DMPQ_ERR_INVALID_ARG, "%s: SKIP needs a cached delta", __func__);
        if (n == 0) return ok();
        return hip_status(launch_tdc_skip(stream, x_in, delta, n, x_out), __func__);
    }
    if (mode != DMPQ_TDC_REFRESH)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown mode %d", __func__, mode);
    REQUIRE_PTR(d_sums4);
    if (dmpq_status s = check_ws(__func__, ws, ws_bytes)) return s;
    return hip_status(launch_tdc_refresh(stream, x_in, x_out, delta, n, delta_valid, d_sums4,
                                         Workspace(ws)),
                      __func__);
}

dmpq_status dmpq_tdc_commit(dmpq_tdc_state *h_st, int mode, const double *h_sums4) {
    REQUIRE_HOST(h_st);
    if (mode == DMPQ_TDC_SKIP) {
        h_st->acc += h_st->d;
        h_st->gamma_valid = 0;
        return ok();
    }
    if (mode != DMPQ_TDC_REFRESH)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown mode %d", __func__, mode);
    REQUIRE_HOST(h_sums4);
    h_st->d = h_st->delta_valid ? rel_ratio(h_sums4[2], h_sums4[3]) : INFINITY;
    h_st->acc = 0.0;
    h_st->n_refresh += 1;
    h_st->delta_valid = 1;
    h_st->gamma = rel_ratio(h_sums4[0], h_sums4[1]);
    h_st->gamma_valid = 1;
    return ok();
}

dmpq_status dmpq_prep_weight(hipStream_t stream, const uint16_t *w, int64_t N, int64_t K,
                             int int8_mode, uint8_t *cw, uint8_t *sw, float *d_gw, int8_t *qw,
                             float *sw_row, void *ws, size_t ws_bytes) {
    if (N < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: N = %lld < 0", __func__, (long long)N);
    if (dmpq_status s = check_k(__func__, K)) return s;
    REQUIRE_PTR_N(w, N);
    REQUIRE_PTR_N(cw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR(d_gw);
    REQUIRE_PTR_N(qw, N);
    REQUIRE_PTR_N(sw_row, N);
    if (int8_mode != DMPQ_W8_FROM_NVFP4 && int8_mode != DMPQ_W8_DIRECT)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown int8_mode %d", __func__, int8_mode);
    if (!hq_int8_supported(K))
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld exceeds 32768", __func__, (long long)K);
    if (dmpq_status s = check_ws(__func__, ws, ws_bytes)) return s;
    hipError_t e = launch_hq_nvfp4(stream, w, N, K, 0, cw, sw, d_gw, Workspace(ws));
    if (e != hipSuccess) return hip_status(e, __func__);
    if (int8_mode == DMPQ_W8_DIRECT)
        e = launch_hq_int8(stream, w, N, K, 0, qw, sw_row);
    else
        e = launch_w8_from_nvfp4(stream, cw, sw, d_gw, N, K, qw, sw_row);
    return hip_status(e, __func__);
}

dmpq_status dmpq_weight_int8_from_nvfp4(hipStream_t stream, const uint8_t *cw, const uint8_t *sw,
                                        const float *d_gw, int64_t N, int64_t K, int8_t *qw,
                                        float *sw_row) {
    if (N < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: N = %lld < 0", __func__, (long long)N);
    if (dmpq_status s = check_k(__func__, K)) return s;
    REQUIRE_PTR_N(cw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR(d_gw);
    REQUIRE_PTR_N(qw, N);
    REQUIRE_PTR_N(sw_row, N);
    if (!hq_int8_supported(K))
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld exceeds 32768", __func__, (long long)K);
    if (N == 0) return ok();
    return hip_status(launch_w8_from_nvfp4(stream, cw, sw, d_gw, N, K, qw, sw_row), __func__);
}

dmpq_status dmpq_hadamard_quant_int8_w8(hipStream_t stream, const uint16_t *x, int64_t M,
                                        int64_t K, int flags, int8_t *q, float *s_row,
                                        const uint8_t *cw, const uint8_t *sw, const float *d_gw,
                                        int64_t N, int8_t *qw, float *sw_row) {
    if (M < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: M = %lld < 0", __func__, (long long)M);
    if (N < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: N = %lld < 0", __func__, (long long)N);
    if (dmpq_status s = check_k(__func__, K)) return s;
    REQUIRE_PTR_N(x, M);
    REQUIRE_PTR_N(q, M);
    REQUIRE_PTR_N(s_row, M);
    REQUIRE_PTR_N(cw, N);
    REQUIRE_PTR_N(sw, N);
    REQUIRE_PTR(d_gw);
    REQUIRE_PTR_N(qw, N);
    REQUIRE_PTR_N(sw_row, N);
    if (flags & ~DMPQ_NO_HADAMARD) return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown flags %d", __func__, flags);
    if (!hq_int8_supported(K))
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld exceeds 32768", __func__, (long long)K);
    return hip_status(launch_hq_int8_w8(stream, x, M, K, flags, q, s_row, cw, sw, d_gw, N, qw, sw_row),
                      __func__);
}

dmpq_status dmpq_outlier_count(hipStream_t stream, const uint16_t *x, int64_t M, int64_t K,
                               double kappa, double *d_count, void *ws, size_t ws_bytes) {
    if (M < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: M = %lld < 0", __func__, (long long)M);
    if (dmpq_status s = check_k(__func__, K)) return s;
    REQUIRE_PTR_N(x, M);
    REQUIRE_PTR(d_count);
    if (!(kappa >= 0.0) || !isfinite(kappa))
        return fail(DMPQ_ERR_INVALID_ARG, "%s: kappa = %g must be finite and >= 0", __func__, kappa);
    if (!hq_int8_supported(K))
        return fail(DMPQ_ERR_UNSUPPORTED, "%s: K = %lld exceeds 32768", __func__, (long long)K);
    if (dmpq_status s = check_ws(__func__, ws, ws_bytes)) return s;
    return hip_status(launch_outlier_count(stream, x, M, K, kappa, d_count, Workspace(ws)), __func__);
}

dmpq_status dmpq_pdr_decide(double h_count, int64_t n, double rho, int *h_force) {
    REQUIRE_HOST(h_force);
    if (n < 0) return fail(DMPQ_ERR_BAD_SHAPE, "%s: n = %lld < 0", __func__, (long long)n);
    *h_force = n > 0 && h_count / (double)n > rho;
    return ok();
}

dmpq_status dmpq_gemm_bf16(hipStream_t stream, const uint16_t *x, const uint16_t *w, int64_t M,
                           int64_t N, int64_t K, int out_dtype, void *y) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    REQUIRE_PTR_N(x, M);
    REQUIRE_PTR_N(w, N);
    REQUIRE_PTR_N(y, M * N);
    if (out_dtype != DMPQ_OUT_F32 && out_dtype != DMPQ_OUT_BF16)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: out_dtype %d is not F32 or BF16", __func__, out_dtype);
    return hip_status(launch_gemm_bf16(stream, x, w, M, N, K, out_dtype, y, 0, nullptr, nullptr),
                      __func__);
}

dmpq_status dmpq_gemm_bf16_ex(hipStream_t stream, const uint16_t *x, const uint16_t *w, int64_t M,
                              int64_t N, int64_t K, int out_dtype, void *y, int epilogue, void *ws,
                              size_t ws_bytes) {
    if (dmpq_status s = check_gemm(__func__, M, N, K)) return s;
    REQUIRE_PTR_N(x, M);
    REQUIRE_PTR_N(w, N);
    REQUIRE_PTR_N(y, M * N);
    if (dmpq_status s = check_epilogue(__func__, M, N, out_dtype, 3, epilogue, ws, ws_bytes)) return s;
    return hip_status(launch_gemm_bf16(stream, x, w, M, N, K, out_dtype, y, epilogue,
                                       static_cast<float *>(ws), split_area(ws, ws_bytes, M, N)),
                      __func__);
}

dmpq_status dmpq_selftest_codec(hipStream_t stream, int codec, uint32_t lo, uint32_t hi,
                                uint32_t *d_stats) {
    if (codec != DMPQ_CODEC_E4M3 && codec != DMPQ_CODEC_E2M1)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: unknown codec %d", __func__, codec);
    if (lo > hi || hi > 0x7F800000u)
        return fail(DMPQ_ERR_INVALID_ARG, "%s: patterns [%u, %u) are not finite non-negative floats",
                    __func__, lo, hi);
    REQUIRE_PTR(d_stats);
    return hip_status(launch_codec_stats(stream, codec, lo, hi, d_stats), __func__);
}

}  // extern "C"
