/*
 * dmpq.h -- C ABI of libdmpq, the MI355X (gfx950) hot path of 6Bit-Diffusion's
 * dynamic mixed-precision quantized linear layer (arXiv 2603.18742).
 *
 * Page citations name the web pages that describe the method:
 *   [gist-en]  gist.science/paper/2603.18742 (English summary)
 *   [gist-it]  gist.science/it/paper/2603.18742 (Italian summary)
 *   [gist-zh]  gist.science/zh/paper/2603.18742 (Chinese technical summary)
 *   [abstract] the paper's English abstract (chatpaper.ai page)
 *
 * Conventions shared by every entry point
 *   - Return value: DMPQ_OK, or an error code; dmpq_last_error() then holds a
 *     message for the calling thread.  No C++ exception crosses this ABI.
 *   - Argument errors are detected and returned before anything is launched.
 *     DMPQ_ERR_HIP means a launch failed; the stream state is then whatever
 *     the HIP runtime reports.
 *   - Pointers prefixed d_ or without prefix are device pointers (GPU memory
 *     of the current device); pointers prefixed h_ are host pointers.  The
 *     caller owns every buffer; the library allocates nothing.
 *   - Device calls are asynchronous and ordered on the given stream (NULL =
 *     the null stream).  Host calls (gate_and_route, tdc_decide, tdc_commit,
 *     tdc_init) are pure functions of their arguments and never touch a GPU.
 *   - Tensors are dense row-major.  bf16 values are passed as uint16_t bit
 *     patterns.  Activations X are [M x K] (row = token, K contiguous);
 *     weights W are [N x K] (row = output channel, K contiguous); Y = X W^T
 *     is [M x N].
 *   - Every device tensor pointer must be 16-byte aligned.  K must be a
 *     positive multiple of 16 (the Hadamard block and the NVFP4 scale group);
 *     the GEMM entry points take K <= 4194304 (2^22; DMPQ_ERR_UNSUPPORTED
 *     beyond).
 *     M, N >= 0 (0 is an empty no-op); a buffer of zero elements may be NULL.
 *   - Non-finite inputs (the pages say nothing of them; the rule taken
 *     here): the quantizers encode a NaN as code 0 (INT8 0, E2M1 +0, E4M3
 *     scale 0) whatever its sign, and a NaN never enters an amax.  An
 *     infinity makes its row's (INT8) or tensor's (NVFP4) amax infinite, so
 *     the reciprocal is 0: scale +inf (INT8 s_row, NVFP4 g), every code 0
 *     and every NVFP4 block scale 0.  The rotation spreads a NaN over its
 *     16-block.  The reductions (Gamma, TDC sums, outlier count) and GEMMs
 *     propagate IEEE results.  Every kernel terminates on any input.
 *   - Workspaces (ws) come from dmpq_workspace_bytes().  They carry
 *     per-workgroup partial results between the kernels of one call and need
 *     no initialization.  Calls that may run concurrently (different streams)
 *     must not share a workspace; calls on one stream may.
 */
#ifndef DMPQ_H
#define DMPQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dmpq_status {
    DMPQ_OK = 0,
    DMPQ_ERR_INVALID_ARG = 1, /* null pointer, unknown enum value */
    DMPQ_ERR_BAD_SHAPE = 2,   /* negative size, K not a multiple of 16, ... */
    DMPQ_ERR_MISALIGNED = 3,  /* a device pointer is not 16-byte aligned */
    DMPQ_ERR_UNSUPPORTED = 4, /* valid but outside what the kernels handle */
    DMPQ_ERR_HIP = 5,         /* the HIP runtime reported an error */
    DMPQ_ERR_WORKSPACE = 6    /* workspace missing or too small */
} dmpq_status;

/* Routes of a linear layer (DMPQ assigns NVFP4 to temporally stable layers,
 * INT8 to volatile ones: [gist-en] §2.A, [abstract]; PDR forces full
 * precision on a refresh whose input has many outliers: [gist-en] §2.C). */
enum { DMPQ_ROUTE_NVFP4 = 0, DMPQ_ROUTE_INT8 = 1, DMPQ_ROUTE_BF16 = 2 };
/* GEMM output types: fp32 (the contract), bf16 (RNE of the fp32 value), and
 * the raw int32 accumulators of the INT8 GEMM (test mode). */
enum { DMPQ_OUT_F32 = 0, DMPQ_OUT_BF16 = 1, DMPQ_OUT_I32 = 2 };
/* Quantizer flags: bit 0 skips the block Hadamard (test hook); bit 1 (NVFP4
 * only) takes the tensor amax from the tile maxima a producer GEMM left in
 * the workspace (DMPQ_EPI_NVFP4_AMAX) instead of reading x for it. */
enum { DMPQ_NO_HADAMARD = 1, DMPQ_AMAX_GIVEN = 2 };
/* Producer epilogues of the *_ex GEMMs (bit flags, BF16 output only):
 * GELU on the way out, and the next linear's NVFP4 tensor-amax term. */
enum { DMPQ_EPI_GELU = 1, DMPQ_EPI_NVFP4_AMAX = 2 };
/* INT8 weight derivation in dmpq_prep_weight. */
enum { DMPQ_W8_FROM_NVFP4 = 0, DMPQ_W8_DIRECT = 1 };
/* TDC step modes. */
enum { DMPQ_TDC_SKIP = 0, DMPQ_TDC_REFRESH = 1 };
/* NVFP4 GEMM variants (both exact; only the fp32 accumulation order differs):
 * 0 = E2M1 x E4M3 products dequantized to 16-bit floats in LDS (exact: at
 *     most 6 significant bits) feeding 16-bit MFMA -- the fast path;
 * 1 = the chip's block-scaled f8f6f4 MFMA on raw E2M1 codes, one 16-element
 *     group per instruction, E4M3 scales applied to the exact group partials
 *     in fp32 (kept for measurement; its power-of-two per-32 scales cannot
 *     carry E4M3 scales inside the instruction). */
enum { DMPQ_FP4_BF16_DEQUANT = 0, DMPQ_FP4_SCALED_MFMA = 1 };
/* Workspace users. */
enum { DMPQ_OP_GAMMA = 0, DMPQ_OP_QUANT_NVFP4 = 1, DMPQ_OP_TDC = 2, DMPQ_OP_PREP_WEIGHT = 3,
       DMPQ_OP_OUTLIER = 4, DMPQ_OP_GEMM_AMAX = 5, DMPQ_OP_GEMM = 6, DMPQ_OP_GEMM_W4 = 7 };

/* Message describing the calling thread's last error ("" if none). */
const char *dmpq_last_error(void);
/* Library version string. */
const char *dmpq_version(void);
/* Bytes of workspace the op needs, 0 for an unknown op.  Most ops need a
 * fixed amount.  Three depend on a GEMM's output shape (pass its M and N as
 * (M, K)): DMPQ_OP_GEMM_AMAX, a fused-amax producer GEMM and the NVFP4
 * quantization of its output; DMPQ_OP_GEMM, the full workspace of the *_ex
 * GEMMs (the same tile maxima first, then 64 MiB for the K split);
 * DMPQ_OP_GEMM_W4, dmpq_qgemm_int8_from_nvfp4 (the tile maxima, then two
 * floats per weight row). */
size_t dmpq_workspace_bytes(int op, int64_t M, int64_t K);

/* ---------------------------------------------------------------------------
 * Gamma predictor sums ([gist-en] §2.A "Mechanism" item 1; [gist-it] §2.A
 * "Meccanismo"): the relative L1 distance between a block's output and input
 * at the previous step.  Writes d_sums2[0] = sum |float(out) - float(in)|
 * (fp32 difference per element) and d_sums2[1] = sum |float(in)|, as fp64,
 * over the n elements of x_in and x_out (bf16).  Gamma = S1/S2 is formed on
 * the host by dmpq_gate_and_route.  Deterministic: the same inputs give the
 * same bits on every call.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_gamma_sums(hipStream_t stream, const uint16_t *x_in, const uint16_t *x_out,
                            int64_t n, double *d_sums2, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * Router ([gist-en] §2.A "Mechanism" items 2-3; [gist-zh] §2.A; missing
 * metric fallback: [gist-en] §2.C "Solution").  Host, pure.
 * h_sums2 = {S1, S2} of the block at the previous step, or NULL when Gamma is
 * missing (first step, or the block was skipped at the previous step).
 * Gamma = S1/S2 (0 if both are 0, +inf if only S2 is 0).  For each of the
 * n_lin linears, E_l = h_alpha[l] * Gamma + h_beta[l] (fp64); route INT8 if
 * E_l > tau, else NVFP4.  Missing Gamma routes every linear to INT8 and
 * writes NaN to h_gamma_out and h_err_out.  h_gamma_out and h_err_out may be
 * NULL; h_route_out has n_lin entries.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_gate_and_route(const double *h_sums2, int n_lin, const double *h_alpha,
                                const double *h_beta, double tau, double *h_gamma_out,
                                double *h_err_out, uint8_t *h_route_out);

/* ---------------------------------------------------------------------------
 * Online block Hadamard + dynamic per-token INT8 quantization ([gist-en]
 * §2.A "Outlier Smoothing" and "Routing"; [gist-zh] §2.A).  For each row of
 * x [M x K] bf16: every 16-element block is rotated by H16/4 (Sylvester
 * order, fp32 butterflies in stages 1, 2, 4, 8, then x0.25); a = max |rotated
 * row|; s_row[m] = a/127; q = RNE(rotated * (127/a)) clamped to +-127; a zero
 * row gives s = 0 and q = 0.  Outputs q [M x K] int8, s_row [M] fp32.
 * flags: DMPQ_NO_HADAMARD skips the rotation.  K <= 32768.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_hadamard_quant_int8(hipStream_t stream, const uint16_t *x, int64_t M,
                                     int64_t K, int flags, int8_t *q, float *s_row);

/* ---------------------------------------------------------------------------
 * Online block Hadamard + dynamic NVFP4 quantization ([gist-en] §1 "Hardware
 * Gap" and §2.A; [gist-it] §3 item 4; [gist-zh] §2.A).  Rotation as above.
 * A = max |rotated tensor| (current tensor, computed on the device);
 * d_g[0] = A/2688 (fp32 tensor scale; 2688 = 6 * 448).  Per 16-block b of a
 * row: scales[m][b] = E4M3(448 * a_b / A) (OCP E4M3FN, RNE, saturating);
 * S = E4M3value * g; codes = E2M1 RNE of rotated * (1/S), sign kept, or +0
 * when S is zero or below FLT_MIN.  codes [M x K/2]: element 2i in the low
 * nibble of byte i; scales [M x K/16] uint8.  A zero tensor gives g = 0 and
 * all-zero outputs.  Two passes over x (tensor amax, then codes).
 * ws: dmpq_workspace_bytes(DMPQ_OP_QUANT_NVFP4, M, K) bytes.
 * flags DMPQ_AMAX_GIVEN: x is the output of a *_ex GEMM with
 * DMPQ_EPI_NVFP4_AMAX, and ws is the workspace that GEMM wrote, untouched
 * since (dmpq_workspace_bytes(DMPQ_OP_GEMM_AMAX, M, K) bytes).  A comes from
 * the GEMM's per-tile maxima, so x is read once; the outputs are the same
 * bits as without the flag.  Not combinable with DMPQ_NO_HADAMARD.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_hadamard_quant_nvfp4(hipStream_t stream, const uint16_t *x, int64_t M,
                                      int64_t K, int flags, uint8_t *codes, uint8_t *scales,
                                      float *d_g, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * dmpq_hadamard_quant_nvfp4 without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * dmpq_hadamard_quant_nvfp4 with flags 0 or DMPQ_NO_HADAMARD; the first
 * pass's partial maxima go to a static 64 KiB device array instead (one copy
 * per device, kept until the process ends; it holds the partials of any
 * tensor size, and a size that would not fit is rejected with
 * DMPQ_ERR_WORKSPACE).  DMPQ_AMAX_GIVEN is rejected (DMPQ_ERR_UNSUPPORTED):
 * it reads the producer GEMM's workspace.  Every argument is checked before
 * the first HIP call (the scratch address is looked up once per device, on
 * the first valid call).  Allocates nothing.  Every call on
 * a device shares that device's array: calls that overlap on one device
 * (concurrent streams, threads) race and must be ordered by the caller.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_hadamard_quant_nvfp4_noalloc(hipStream_t stream, const uint16_t *x, int64_t M,
                                              int64_t K, int flags, uint8_t *codes,
                                              uint8_t *scales, float *d_g);

/* ---------------------------------------------------------------------------
 * INT8 quantized linear ([gist-en] §2.A "Routing"; [gist-zh] §2.A weight
 * handling).  acc[m][n] = sum_k qa[m][k] * qw[n][k] (exact int32: codes in
 * [-127, 127] keep |acc| < 2^31 for any K <= 133144; beyond that the int32
 * sum wraps if the products do not cancel), then
 * out_dtype F32: y = (float(acc) * sa[m]) * sw[n]; BF16: RNE of that value;
 * I32: the accumulator.  qa [M x K] int8 with per-row scales sa [M];
 * qw [N x K] int8 with per-output-channel scales sw [N]; y [M x N].
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_qgemm_int8(hipStream_t stream, const int8_t *qa, const float *sa,
                            const int8_t *qw, const float *sw, int64_t M, int64_t N, int64_t K,
                            int out_dtype, void *y);

/* ---------------------------------------------------------------------------
 * NVFP4 quantized linear ([gist-en] §1 and §3 item 4; [gist-zh] §2.A).
 * y[m][n] = ga * gw * sum_b eA[m][b] eW[n][b] sum_{k in b} vA[m][k] vW[n][k],
 * accumulated in fp32 (every product E2M1 x E4M3 is exact; only the fp32
 * accumulation rounds).  ca/sa/d_ga: activation codes [M x K/2], E4M3
 * scales [M x K/16], tensor scale (device fp32); cw/sw/d_gw likewise for the
 * weight [N x K].  out_dtype F32 or BF16.  variant: DMPQ_FP4_BF16_DEQUANT or
 * DMPQ_FP4_SCALED_MFMA.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_qgemm_nvfp4(hipStream_t stream, const uint8_t *ca, const uint8_t *sa,
                             const float *d_ga, const uint8_t *cw, const uint8_t *sw,
                             const float *d_gw, int64_t M, int64_t N, int64_t K,
                             int out_dtype, void *y, int variant);

/* ---------------------------------------------------------------------------
 * Temporal Delta Cache ([gist-en] §2.B; [gist-it] §2.B; [gist-zh] §2.B).
 * Host state of one block; the cached delta itself is a caller-owned device
 * bf16 buffer of the block's activation size.
 * ------------------------------------------------------------------------- */
typedef struct dmpq_tdc_state {
    int64_t n_refresh;   /* computed (refreshed) steps so far */
    double d;            /* relative L1 distance of the last two deltas (+inf until two exist) */
    double acc;          /* accumulated error of the current run of skips */
    int32_t delta_valid; /* the device delta buffer holds a delta */
    int32_t gamma_valid; /* gamma holds the Gamma of the last step (0 after a skip) */
    double gamma;        /* S1/S2 of the last computed step */
} dmpq_tdc_state;

typedef struct dmpq_tdc_params {
    double eps_sim;   /* skip only if d < eps_sim (deltas similar enough) */
    double delta_acc; /* ... and acc + d <= delta_acc (accumulated-error gate) */
} dmpq_tdc_params;

/* Fresh state: no delta, d = +inf, acc = 0, Gamma missing.  Host. */
dmpq_status dmpq_tdc_init(dmpq_tdc_state *h_st);

/* Skip decision, host, pure: *h_skip = 1 iff n_refresh >= 2 and a delta is
 * cached and d < eps_sim and acc + d <= delta_acc. */
dmpq_status dmpq_tdc_decide(const dmpq_tdc_state *h_st, const dmpq_tdc_params *h_p,
                            int *h_skip);

/* Device step over n bf16 elements.
 * SKIP: x_out = bf16(float(x_in) + float(delta)) (the cached delta is reused;
 *   d_sums4, ws unused and may be NULL).
 * REFRESH (x_out = the block's computed output): new = bf16(out - in);
 *   d_sums4 = {S1 = sum |out - in| (fp32 difference), S2 = sum |in|,
 *   S3 = sum |new - delta|, S4 = sum |delta|} in fp64, S3 = S4 = 0 when
 *   delta_valid is 0; then delta <- new.  ws: DMPQ_OP_TDC workspace. */
dmpq_status dmpq_tdc_step(hipStream_t stream, int mode, const uint16_t *x_in, uint16_t *x_out,
                          uint16_t *delta, int64_t n, int delta_valid, double *d_sums4,
                          void *ws, size_t ws_bytes);

/* Host bookkeeping after a step.  SKIP: acc += d, Gamma becomes missing.
 * REFRESH (h_sums4 = the step's sums, copied to the host): d = S3/S4 if a
 * delta was cached before (0 if both 0, +inf if only S4 is 0), else +inf;
 * acc = 0; n_refresh += 1; delta_valid = 1; gamma = S1/S2, gamma_valid = 1. */
dmpq_status dmpq_tdc_commit(dmpq_tdc_state *h_st, int mode, const double *h_sums4);

/* ---------------------------------------------------------------------------
 * Offline weight preparation ([gist-zh] §2.A weight-handling bullet: weights
 * are quantized to NVFP4 offline and converted when an INT8 GEMM needs
 * them).  w [N x K] bf16 is block-rotated like the activations, then
 * quantized to NVFP4 exactly as dmpq_hadamard_quant_nvfp4 (cw, sw, d_gw).
 * INT8 weight qw [N x K] with per-row scales sw_row [N]:
 *   DMPQ_W8_FROM_NVFP4: wd = (E2M1value * E4M3value) * gw, then per row
 *     s = amax/127, q = RNE(wd * (127/amax)) clamped to +-127;
 *   DMPQ_W8_DIRECT: dmpq_hadamard_quant_int8 of w.
 * ws: DMPQ_OP_PREP_WEIGHT workspace.  Runs once per weight, off the hot path.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_prep_weight(hipStream_t stream, const uint16_t *w, int64_t N, int64_t K,
                             int int8_mode, uint8_t *cw, uint8_t *sw, float *d_gw, int8_t *qw,
                             float *sw_row, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * INT8 weight from the NVFP4 weight, when an INT8-routed linear needs it
 * ([gist-zh] §2.A weight-handling bullet: weights are kept in NVFP4 and
 * converted for the INT8 GEMM).  With it a model stores only the 4.5-bit
 * weights and converts one linear's weight into a scratch INT8 buffer right
 * before its INT8 GEMM.  Same rule as DMPQ_W8_FROM_NVFP4 of dmpq_prep_weight
 * (bit-identical output): wd = (E2M1value * E4M3value) * gw, per row
 * s = amax/127, q = RNE(wd * (127/amax)) clamped to +-127; a row whose
 * 127/amax is not finite gets s = 0 and q = 0.
 * cw [N x K/2], sw [N x K/16] E4M3, d_gw fp32 (device) -> qw [N x K] int8,
 * sw_row [N] fp32.  K % 16 == 0, K <= 32768.  Stream-ordered; no workspace.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_weight_int8_from_nvfp4(hipStream_t stream, const uint8_t *cw, const uint8_t *sw,
                                        const float *d_gw, int64_t N, int64_t K, int8_t *qw,
                                        float *sw_row);

/* ---------------------------------------------------------------------------
 * The two row quantizations of an INT8-routed linear in one launch: the
 * activation quantization of dmpq_hadamard_quant_int8 (x, M, K, flags -> q,
 * s_row) and the weight conversion of dmpq_weight_int8_from_nvfp4 (cw, sw,
 * d_gw, N, K -> qw, sw_row), for the same K ([gist-en] §2.A "Routing": INT8
 * activations per token; [gist-zh] §2.A weight-handling bullet: the NVFP4
 * weight converted when an INT8 GEMM needs it).  Outputs are bit-identical
 * to the two separate calls; M or N may be 0 (that half is skipped).
 * Argument rules and errors as the two calls; no workspace.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_hadamard_quant_int8_w8(hipStream_t stream, const uint16_t *x, int64_t M,
                                        int64_t K, int flags, int8_t *q, float *s_row,
                                        const uint8_t *cw, const uint8_t *sw, const float *d_gw,
                                        int64_t N, int8_t *qw, float *sw_row);

/* ---------------------------------------------------------------------------
 * INT8 linear against an NVFP4 weight converted inside the GEMM ([gist-zh]
 * §2.A weight-handling bullet: weights stay in NVFP4 and are converted when
 * an INT8 GEMM needs them).  No INT8 copy of the weight is written: a first
 * kernel computes each weight row's scale s_row = amax/127 and reciprocal
 * 127/amax (the rule of dmpq_weight_int8_from_nvfp4) into ws, and the GEMM
 * requantizes each weight tile from the NVFP4 codes as it stages the tile.
 * y equals dmpq_qgemm_int8_ex(qa, sa, qw, sw_row, ...) with (qw, sw_row) from
 * dmpq_weight_int8_from_nvfp4(cw, sw, d_gw), bit for bit, on every output
 * type and epilogue.  qa [M x K] int8, sa [M]; cw [N x K/2], sw [N x K/16],
 * d_gw (device fp32).  K % 128 == 0 (else DMPQ_ERR_UNSUPPORTED).  out_dtype
 * F32, BF16 or I32; epilogue as dmpq_qgemm_int8_ex (no tail split).  ws:
 * dmpq_workspace_bytes(DMPQ_OP_GEMM_W4, M, N) bytes, required; calls that
 * share a workspace must not overlap.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_qgemm_int8_from_nvfp4(hipStream_t stream, const int8_t *qa, const float *sa,
                                       const uint8_t *cw, const uint8_t *sw, const float *d_gw,
                                       int64_t M, int64_t N, int64_t K, int out_dtype, void *y,
                                       int epilogue, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * Purified Delta Refresh ([gist-en] §2.C "Solution"; [gist-it] §2.C;
 * [gist-zh] §2.C): before a refresh writes a block's delta into the cache,
 * the block input is checked for outliers; a high outlier ratio computes the
 * block's linears in full precision (BF16) for that step, so the cached delta
 * carries no quantization noise.  The pages define neither "outlier" nor the
 * threshold; this library's reading:
 *   an element x of token row m (K channels, raw input) is an outlier when
 *   x^2 * K > kappa^2 * S_m, S_m = sum_k x_k^2, all in fp64 (|x| above kappa
 *   times the row's RMS); the block is forced to BF16 when
 *   count / (M K) > rho (strictly).
 *
 * Device count: x [M x K] bf16 -> *d_count (fp64, an exact integer).  S_m is
 * added in a fixed order, so the result is deterministic; it can differ from
 * a differently ordered sum only for elements within about 1e-15 relative of
 * the threshold.  K % 16 == 0, K <= 32768.  ws: DMPQ_OP_OUTLIER workspace.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_outlier_count(hipStream_t stream, const uint16_t *x, int64_t M, int64_t K,
                               double kappa, double *d_count, void *ws, size_t ws_bytes);

/* Host decision: *h_force = 1 when n > 0 and h_count / n > rho, else 0. */
dmpq_status dmpq_pdr_decide(double h_count, int64_t n, double rho, int *h_force);

/* Full-precision linear of the PDR route: y[m,n] = sum_k x[m,k] w[n,k] over
 * bf16 operands (x [M x K], w [N x K] = the original, unrotated bf16 weight),
 * exact products, fp32 accumulation in an unspecified order.  out_dtype F32
 * or BF16 (RNE of the fp32 value).  K % 16 == 0; any M, N >= 0. */
dmpq_status dmpq_gemm_bf16(hipStream_t stream, const uint16_t *x, const uint16_t *w, int64_t M,
                           int64_t N, int64_t K, int out_dtype, void *y);

/* ---------------------------------------------------------------------------
 * Producer-fused epilogues: the three linears above with an epilogue that
 * prepares the next linear's input ([gist-en] §2.A "Outlier Smoothing": the
 * rotation must cost little, so its tensor-wide pass is folded into the GEMM
 * that produces the tensor).  out_dtype must be DMPQ_OUT_BF16 when
 * epilogue != 0.
 *   DMPQ_EPI_GELU: y = bf16(GELU(float(bf16(v)))) for the linear's value v,
 *     GELU(u) = u * Phi(u) = u/2 * erfc(-u/sqrt 2) in fp32 -- the same result
 *     as a separate bf16 GELU after the GEMM, up to GELU's own rounding.
 *   DMPQ_EPI_NVFP4_AMAX: the kernel also writes, per 256 x 256 output tile,
 *     max |H16 rotation of its 16-blocks| over the stored y (the rotation and
 *     fp32 order of dmpq_hadamard_quant_nvfp4) into ws, for a following
 *     dmpq_hadamard_quant_nvfp4(y, M, N, DMPQ_AMAX_GIVEN, ..., ws).  Needs
 *     N % 16 == 0 and ws of dmpq_workspace_bytes(DMPQ_OP_GEMM_AMAX, M, N)
 *     bytes; ws may be NULL otherwise.
 * The NVFP4 variant is always DMPQ_FP4_BF16_DEQUANT.
 *
 * Tail split: with ws of dmpq_workspace_bytes(DMPQ_OP_GEMM, M, N) bytes, the
 * last partial wave of 256 x 256 tiles (the tiles beyond the last multiple
 * of 256) is split along K over otherwise idle CUs, and a second kernel adds
 * each tile's parts in a fixed order before the epilogue.  INT8 results are
 * unchanged; NVFP4 and BF16 results differ from the unsplit ones only in the
 * fp32 summation order (deterministic, within the same tolerance).  Applies
 * on the DMA paths (INT8 K % 128 == 0 and K >= 4096, NVFP4 K % 128 == 0
 * and K >= 256, every BF16 K) and not to the INT8 I32 output.  Calls that
 * share a workspace must not overlap.
 * epilogue 0 with ws NULL is the plain call.
 * ------------------------------------------------------------------------- */
dmpq_status dmpq_qgemm_int8_ex(hipStream_t stream, const int8_t *qa, const float *sa,
                               const int8_t *qw, const float *sw, int64_t M, int64_t N, int64_t K,
                               int out_dtype, void *y, int epilogue, void *ws, size_t ws_bytes);
dmpq_status dmpq_qgemm_nvfp4_ex(hipStream_t stream, const uint8_t *ca, const uint8_t *sa,
                                const float *d_ga, const uint8_t *cw, const uint8_t *sw,
                                const float *d_gw, int64_t M, int64_t N, int64_t K,
                                int out_dtype, void *y, int epilogue, void *ws, size_t ws_bytes);
dmpq_status dmpq_gemm_bf16_ex(hipStream_t stream, const uint16_t *x, const uint16_t *w, int64_t M,
                              int64_t N, int64_t K, int out_dtype, void *y, int epilogue, void *ws,
                              size_t ws_bytes);

/* ---------------------------------------------------------------------------
 * Self-test of the device converters behind the quantizers ([gist-en] §1:
 * NVFP4 codes are E2M1 with E4M3 block scales).  Not on the hot path.
 * codec DMPQ_CODEC_E4M3: the block-scale encoder on non-negative inputs
 *   (nearest E4M3, ties to even, saturating at 448); DMPQ_CODEC_E2M1: the
 *   element converter (nearest E2M1, ties to even, saturating at 6, sign
 *   kept) on +f and -f.  Over the fp32 bit patterns p in [lo, hi)
 *   (0 <= lo <= hi <= 0x7F800000, i.e. finite non-negative floats f), for
 *   each code c writes d_stats[3c] = the lowest p encoding to c (0xFFFFFFFF
 *   if none), d_stats[3c+1] = the highest, d_stats[3c+2] = how many (codes
 *   0..127 for E4M3; 0..15 for E2M1, the negated inputs in 8..15).  Both
 *   converters are monotone in p, so these equal a reference encoder's
 *   exactly when every pattern agrees.  d_stats: 384 (E4M3) or 48 (E2M1)
 *   uint32, device.
 * ------------------------------------------------------------------------- */
enum { DMPQ_CODEC_E4M3 = 0, DMPQ_CODEC_E2M1 = 1 };
dmpq_status dmpq_selftest_codec(hipStream_t stream, int codec, uint32_t lo, uint32_t hi,
                                uint32_t *d_stats);

#ifdef __cplusplus
}
#endif
#endif /* DMPQ_H */
