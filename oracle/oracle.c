/*
 * oracle.c -- plain, slow CPU reference for the dynamic mixed-precision
 * quantized linear layer of 6Bit-Diffusion.  TEST INFRASTRUCTURE ONLY (see
 * oracle.h for who may call it and for the page-citation short names).
 *
 * Written for readability, not speed: codecs are nearest-value searches over
 * the format's value set, the Hadamard is the textbook butterfly, GEMMs are
 * triple loops.  OpenMP only splits independent rows; it never changes an
 * arithmetic result.  Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp.
 */
#include "oracle.h"

#include <float.h>
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

int orc_max_threads(void)
{
    return omp_get_max_threads();
}

void orc_set_threads(int n)
{
    if (n > 0)
        omp_set_num_threads(n);
}

/* ======================================================================
 * Codecs.  The pages name the formats only: NVFP4 is a micro-scaling block
 * format whose elements are E2M1 ([gist-it] §4 "Supporto Hardware Nativo";
 * [gist-en] §1 "Hardware Gap"), with one E4M3 scale per 16 elements and an
 * fp32 tensor scale.  Values follow the OCP 8-bit / microscaling format
 * specifications: E2M1 = 1 sign, 2 exponent (bias 1), 1 mantissa bit, no
 * inf/NaN; E4M3 (FN variant) = 1 sign, 4 exponent (bias 7), 3 mantissa bits,
 * max 448, only S.1111.111 is NaN.
 * ==================================================================== */

uint16_t orc_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return 0x7FC0; /* canonical quiet NaN */
    /* round to nearest, ties to even, on the 16 dropped bits */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float orc_e2m1_value(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    float mag = (e == 0) ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
    return s ? -mag : mag;
}

uint8_t orc_e2m1_encode(float v)
{
    /* E2M1 has no NaN, and the pages say nothing of non-finite inputs.  The
     * rule taken here: a NaN encodes as +0 whatever its sign bit (CPUs and
     * GPUs give invalid operations NaNs of different signs, so a rule that
     * kept the sign would not be portable). */
    if (isnan(v))
        return 0;
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs((double)v);
    if (a >= 6.0)
        return sign | 7; /* saturate to the largest magnitude */
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; c++) {
        double d = fabs(a - (double)orc_e2m1_value((uint8_t)c));
        /* scanning upward, a tie is always between c-1 and c: keep the even one */
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            bestd = d;
            best = c;
        }
    }
    return sign | (uint8_t)best;
}

float orc_e4m3_value(uint8_t code)
{
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    float mag = (e == 0) ? ldexpf((float)m, -9) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return s ? -mag : mag;
}

uint8_t orc_e4m3_encode(float v)
{
    /* block scales are non-negative by construction; callers pass v >= 0.
     * A NaN (the ratio Inf/Inf of a block holding an infinity when the
     * tensor amax is infinite) encodes as 0, a zero scale. */
    if (isnan(v))
        return 0;
    double a = (double)v;
    if (a >= 448.0)
        return 0x7E; /* saturate to the largest finite value */
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        double d = fabs(a - (double)orc_e4m3_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            bestd = d;
            best = c;
        }
    }
    return (uint8_t)best;
}

/* ======================================================================
 * Online block Hadamard.  The pages apply a fast Hadamard transform to local
 * blocks of each activation row to spread outliers ([gist-en] §2.A "Outlier
 * Smoothing"; [gist-zh] §2.A, outlier smoothing bullet).  Block size 16
 * (the pages give none; 16 matches the NVFP4 scale group), Sylvester order,
 * butterfly stages h = 1, 2, 4, 8 in fp32, then one exact scaling by 1/4 so
 * the transform is orthonormal: out = (H16 / 4) * in.
 * ==================================================================== */

void orc_fwht16(const float in[16], float out[16])
{
    float v[16];
    for (int i = 0; i < 16; i++)
        v[i] = in[i];
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; i++)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
    for (int i = 0; i < 16; i++)
        out[i] = v[i] * 0.25f;
}

/* one row of bf16 -> fp32, rotated block by block unless flags say not to */
static void rotate_row(const uint16_t *x, int64_t K, int flags, float *out)
{
    for (int64_t k = 0; k < K; k++)
        out[k] = orc_bf16_value(x[k]);
    if (flags & ORC_NO_HADAMARD)
        return;
    for (int64_t j = 0; j < K; j += 16)
        orc_fwht16(out + j, out + j);
}

static int bad_shape(int64_t M, int64_t K)
{
    return M < 0 || K <= 0 || (K % 16) != 0;
}

/* ======================================================================
 * Dynamic INT8 activation quantization, per token (row), symmetric, on the
 * rotated row.  INT8 is the route for volatile layers ([gist-en] §2.A
 * "Routing"; [gist-it] §2.A "Routing Dinamico").  Range +-127, scale =
 * amax/127, codes = RNE(x * (127/amax)).  A row whose 127/amax is not a
 * finite fp32 (amax zero, or below about 3.7e-37) gets scale 0 and zero
 * codes.
 * ==================================================================== */

/* A rounded product as an INT8 code: clamped to +-127; a NaN product (a NaN
 * input, or an infinity times the zero reciprocal of an infinite row amax)
 * codes 0.  The amax ignores NaNs, so they never change a row's scale; a row
 * holding an infinity gets scale +inf and all codes 0. */
static int8_t int8_code(float r)
{
    if (isnan(r))
        return 0;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

int orc_quant_int8(const uint16_t *x, int64_t M, int64_t K, int flags,
                   int8_t *q, float *s_row)
{
    if (bad_shape(M, K))
        return -1;
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; m++) {
            rotate_row(x + m * K, K, flags, row);
            float a = 0.0f;
            for (int64_t k = 0; k < K; k++)
                if (fabsf(row[k]) > a)
                    a = fabsf(row[k]);
            float inv = 127.0f / a;
            if (a == 0.0f || isinf(inv)) { /* no finite reciprocal: a zero row */
                s_row[m] = 0.0f;
                for (int64_t k = 0; k < K; k++)
                    q[m * K + k] = 0;
                continue;
            }
            s_row[m] = a / 127.0f;
            for (int64_t k = 0; k < K; k++)
                q[m * K + k] = int8_code(rintf(row[k] * inv));
        }
        free(row);
    }
    return 0;
}

/* ======================================================================
 * Dynamic NVFP4 activation quantization (current-tensor amax, computed
 * online).  Two-level scaling: the fp32 tensor scale g maps the rotated
 * tensor's absmax A to 6 * 448 (largest E2M1 times largest E4M3); each
 * 16-element block stores the E4M3 code of 448 * a_b / A, so its dequant
 * scale S = E4M3(448 a_b / A) * g is close to a_b / 6.  Codes are the E2M1
 * RNE of x * (1/S).  A block whose S is zero or below the fp32 normal
 * range (where 1/S could overflow) stores +0 codes.  Packing: element 2i in
 * the low nibble of byte i, element 2i+1 in the high nibble; scales are
 * row-major [M][K/16].
 * ==================================================================== */

int orc_quant_nvfp4(const uint16_t *x, int64_t M, int64_t K, int flags,
                    uint8_t *codes, uint8_t *scales, float *g)
{
    if (bad_shape(M, K))
        return -1;
    const int64_t nb = K / 16;

    /* pass 1: tensor amax of the rotated tensor (max is order independent) */
    float A = 0.0f;
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
        float a_loc = 0.0f;
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; m++) {
            rotate_row(x + m * K, K, flags, row);
            for (int64_t k = 0; k < K; k++)
                if (fabsf(row[k]) > a_loc)
                    a_loc = fabsf(row[k]);
        }
#pragma omp critical
        if (a_loc > A)
            A = a_loc;
        free(row);
    }

    if (A == 0.0f) {
        *g = 0.0f;
        memset(scales, 0, (size_t)(M * nb));
        memset(codes, 0, (size_t)(M * K / 2));
        return 0;
    }
    const float gt = A / 2688.0f;
    *g = gt;

    /* pass 2: block scales and codes */
#pragma omp parallel
    {
        float *row = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; m++) {
            rotate_row(x + m * K, K, flags, row);
            for (int64_t b = 0; b < nb; b++) {
                const float *blk = row + 16 * b;
                float ab = 0.0f;
                for (int i = 0; i < 16; i++)
                    if (fabsf(blk[i]) > ab)
                        ab = fabsf(blk[i]);
                float r = ab / A;
                uint8_t e = orc_e4m3_encode(r * 448.0f);
                float S = orc_e4m3_value(e) * gt;
                scales[m * nb + b] = e;
                uint8_t c[16];
                if (!(S >= FLT_MIN)) {
                    memset(c, 0, sizeof c);
                } else {
                    float inv = 1.0f / S;
                    for (int i = 0; i < 16; i++)
                        c[i] = orc_e2m1_encode(blk[i] * inv);
                }
                uint8_t *dst = codes + m * (K / 2) + 8 * b;
                for (int i = 0; i < 8; i++)
                    dst[i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
            }
        }
        free(row);
    }
    return 0;
}

/* ======================================================================
 * Offline weight preparation.  All weights are quantized to NVFP4 offline;
 * an INT8-routed linear needs its weight converted to INT8 for the GEMM
 * ([gist-zh] §2.A, weight-handling bullet).  Weights carry the same block
 * rotation as the activations, since (X H)(W H)^T = X W^T for orthonormal
 * H.  INT8 weight, mode FROM_NVFP4: dequantize the NVFP4 weight,
 * wd = (value * blockscale) * g, then per output channel absmax requant
 * (scale = amax/127, codes RNE(wd * (127/amax))).  Mode DIRECT: per output
 * channel INT8 quant of the rotated bf16 weight (same rule as activations).
 * ==================================================================== */

int orc_w8_from_nvfp4(const uint8_t *cw, const uint8_t *sw, const float *gw,
                      int64_t N, int64_t K, int8_t *qw, float *sw_row)
{
    if (bad_shape(N, K))
        return -1;
    const int64_t nb = K / 16;
    const float g = *gw;
#pragma omp parallel
    {
        float *wd = (float *)malloc((size_t)K * sizeof(float));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; n++) {
            float a = 0.0f;
            for (int64_t k = 0; k < K; k++) {
                uint8_t byte = cw[n * (K / 2) + k / 2];
                uint8_t c = (k & 1) ? (byte >> 4) : (byte & 15);
                float s = orc_e4m3_value(sw[n * nb + k / 16]);
                wd[k] = (orc_e2m1_value(c) * s) * g;
                if (fabsf(wd[k]) > a)
                    a = fabsf(wd[k]);
            }
            float inv = 127.0f / a;
            if (a == 0.0f || isinf(inv)) {
                sw_row[n] = 0.0f;
                for (int64_t k = 0; k < K; k++)
                    qw[n * K + k] = 0;
                continue;
            }
            sw_row[n] = a / 127.0f;
            for (int64_t k = 0; k < K; k++)
                qw[n * K + k] = int8_code(rintf(wd[k] * inv));
        }
        free(wd);
    }
    return 0;
}

int orc_prep_weight(const uint16_t *w, int64_t N, int64_t K, int int8_mode,
                    uint8_t *cw, uint8_t *sw, float *gw,
                    int8_t *qw, float *sw_row)
{
    if (bad_shape(N, K))
        return -1;
    if (orc_quant_nvfp4(w, N, K, 0, cw, sw, gw) != 0)
        return -1;
    if (int8_mode == ORC_W8_DIRECT)
        return orc_quant_int8(w, N, K, 0, qw, sw_row);
    if (int8_mode != ORC_W8_FROM_NVFP4)
        return -1;
    return orc_w8_from_nvfp4(cw, sw, gw, N, K, qw, sw_row);
}

/* ======================================================================
 * Quantized linear layer, Y = X W^T at the routed precision.
 * INT8: exact int32 dot products, then y = (float(acc) * sA[m]) * sW[n].
 * NVFP4: y = gA gW sum_b eA[m,b] eW[n,b] sum_{k in b} vA vW, evaluated in
 * fp64 (every per-block term is exact), plus the summation-scale bound
 * B = gA gW sum_k |a_k| |w_k| used for the fp32 tolerance.
 * ==================================================================== */

int orc_gemm_int8(const int8_t *qa, const float *sa, const int8_t *qw,
                  const float *sw, int64_t M, int64_t N, int64_t K,
                  const int64_t *rows, int64_t n_rows,
                  int32_t *acc, float *y)
{
    if (M < 0 || N < 0 || K <= 0)
        return -1;
    const int64_t R = rows ? n_rows : M;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t i = 0; i < R; i++) {
        int64_t m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            err = 1;
            continue;
        }
        for (int64_t n = 0; n < N; n++) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; k++)
                s += (int64_t)qa[m * K + k] * (int64_t)qw[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) {
                err = 1;
                continue;
            }
            int32_t a32 = (int32_t)s;
            if (acc)
                acc[i * N + n] = a32;
            if (y)
                y[i * N + n] = ((float)a32 * sa[m]) * sw[n];
        }
    }
    return err ? -1 : 0;
}

static float nibble_value(const uint8_t *codes, int64_t rowlen_bytes, int64_t r, int64_t k)
{
    uint8_t byte = codes[r * rowlen_bytes + k / 2];
    return orc_e2m1_value((k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15));
}

int orc_gemm_nvfp4(const uint8_t *ca, const uint8_t *sa, float ga,
                   const uint8_t *cw, const uint8_t *sw, float gw,
                   int64_t M, int64_t N, int64_t K,
                   const int64_t *rows, int64_t n_rows,
                   double *y, double *bound)
{
    if (M < 0 || N < 0 || K <= 0 || (K % 16) != 0)
        return -1;
    const int64_t R = rows ? n_rows : M;
    const int64_t nb = K / 16;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t i = 0; i < R; i++) {
        int64_t m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            err = 1;
            continue;
        }
        for (int64_t n = 0; n < N; n++) {
            double sum = 0.0, babs = 0.0;
            for (int64_t b = 0; b < nb; b++) {
                double ea = orc_e4m3_value(sa[m * nb + b]);
                double ew = orc_e4m3_value(sw[n * nb + b]);
                double inner = 0.0, inner_abs = 0.0;
                for (int64_t k = 16 * b; k < 16 * b + 16; k++) {
                    double p = (double)nibble_value(ca, K / 2, m, k) *
                               (double)nibble_value(cw, K / 2, n, k);
                    inner += p;
                    inner_abs += fabs(p);
                }
                sum += (ea * ew) * inner;
                babs += (ea * ew) * inner_abs;
            }
            if (y)
                y[i * N + n] = (sum * (double)ga) * (double)gw;
            if (bound)
                bound[i * N + n] = (babs * (double)ga) * (double)gw;
        }
    }
    return err ? -1 : 0;
}

/* ======================================================================
 * Gamma predictor: relative L1 distance between a block's output and input
 * at the previous step ([gist-en] §2.A "Mechanism"; [gist-it] §2.A
 * "Meccanismo").  Base of "relative": the L1 norm of the input.
 * S1 = sum |float(out) - float(in)| (fp32 difference, fp64 sum),
 * S2 = sum |float(in)|, Gamma = S1/S2; S2 = 0 gives 0 (S1 = 0) or +inf.
 * ==================================================================== */

void orc_gamma_sums(const uint16_t *x_in, const uint16_t *x_out, int64_t n,
                    double sums[2])
{
    double s1 = 0.0, s2 = 0.0;
    for (int64_t i = 0; i < n; i++) {
        float a = orc_bf16_value(x_in[i]);
        float b = orc_bf16_value(x_out[i]);
        float d = b - a;
        s1 += fabsf(d);
        s2 += fabsf(a);
    }
    sums[0] = s1;
    sums[1] = s2;
}

static double rel_ratio(double num, double den)
{
    if (den == 0.0)
        return num == 0.0 ? 0.0 : INFINITY;
    return num / den;
}

double orc_gamma(const double sums[2])
{
    return rel_ratio(sums[0], sums[1]);
}

/* Router: predicted error E_l = alpha_l * Gamma + beta_l from the pre-fitted
 * linear model; E_l above tau (strictly) sends linear l to INT8, otherwise
 * NVFP4 ([gist-en] §2.A "Mechanism" items 2-3).  A block whose Gamma is
 * missing (first step, or skipped at the previous step) falls back to INT8
 * for every linear ([gist-en] §2.C "Solution", second bullet). */
void orc_route(const double *sums, int n_lin, const double *alpha,
               const double *beta, double tau, double *gamma_out,
               double *err_out, uint8_t *route_out)
{
    double gm = sums ? orc_gamma(sums) : NAN;
    if (gamma_out)
        *gamma_out = gm;
    for (int l = 0; l < n_lin; l++) {
        if (!sums) {
            if (err_out)
                err_out[l] = NAN;
            route_out[l] = ORC_ROUTE_INT8;
            continue;
        }
        double e = alpha[l] * gm + beta[l];
        if (err_out)
            err_out[l] = e;
        route_out[l] = (e > tau) ? ORC_ROUTE_INT8 : ORC_ROUTE_NVFP4;
    }
}

/* ======================================================================
 * Temporal Delta Cache ([gist-en] §2.B; [gist-it] §2.B; [gist-zh] §2.B).
 * The block's residual delta is out - in.  After a computed step, d is the
 * relative L1 distance between the new delta and the previous one (small d
 * = similar).  A block is skipped when two deltas exist, d < eps_sim, and
 * the accumulated error including this skip stays within delta_acc; a skip
 * outputs in + cached delta and adds d to the accumulated error; a computed
 * step resets it.  The delta is cached in bf16.
 * ==================================================================== */

void orc_tdc_init(orc_tdc_state *st)
{
    memset(st, 0, sizeof *st);
    st->d = INFINITY;
}

int orc_tdc_decide(const orc_tdc_state *st, double eps_sim, double delta_acc)
{
    if (st->n_refresh < 2 || !st->delta_valid)
        return 0;
    if (!(st->d < eps_sim))
        return 0;
    if (!(st->acc + st->d <= delta_acc))
        return 0;
    return 1;
}

void orc_tdc_skip(const uint16_t *x_in, const uint16_t *delta, int64_t n,
                  uint16_t *x_out)
{
    for (int64_t i = 0; i < n; i++)
        x_out[i] = orc_bf16_round(orc_bf16_value(x_in[i]) + orc_bf16_value(delta[i]));
}

void orc_tdc_refresh(const uint16_t *x_in, const uint16_t *x_out,
                     uint16_t *delta, int64_t n, int delta_valid,
                     double sums[4])
{
    double s1 = 0.0, s2 = 0.0, s3 = 0.0, s4 = 0.0;
    for (int64_t i = 0; i < n; i++) {
        float a = orc_bf16_value(x_in[i]);
        float b = orc_bf16_value(x_out[i]);
        float dn = b - a;
        uint16_t dnb = orc_bf16_round(dn);
        s1 += fabsf(dn);
        s2 += fabsf(a);
        if (delta_valid) {
            float dp = orc_bf16_value(delta[i]);
            s3 += fabsf(orc_bf16_value(dnb) - dp);
            s4 += fabsf(dp);
        }
        delta[i] = dnb;
    }
    sums[0] = s1;
    sums[1] = s2;
    sums[2] = s3;
    sums[3] = s4;
}

void orc_tdc_commit_skip(orc_tdc_state *st)
{
    st->acc += st->d;
    st->gamma_valid = 0;
}

void orc_tdc_commit_refresh(orc_tdc_state *st, const double sums[4])
{
    st->d = st->delta_valid ? rel_ratio(sums[2], sums[3]) : INFINITY;
    st->acc = 0.0;
    st->n_refresh += 1;
    st->delta_valid = 1;
    st->gamma = rel_ratio(sums[0], sums[1]);
    st->gamma_valid = 1;
}

/* ======================================================================
 * Purified Delta Refresh ([gist-en] §2.C "Solution"; [gist-it] §2.C;
 * [gist-zh] §2.C).  Before a refresh writes a block's delta into the cache,
 * the block input is checked for outliers; a high outlier ratio computes the
 * block's linears in full precision (BF16 operands, fp32 accumulation, no
 * quantization) for that step, so the cached delta carries no quantization
 * noise.  The pages do not define "outlier": here an element x of token row
 * m (K channels) is an outlier when |x| > kappa * RMS(row m), tested exactly
 * as x^2 * K > (kappa * kappa) * S_m with S_m = sum_k x_k^2 in fp64 (the
 * square of a bf16 value is exact in fp64).  The ratio is outliers / (M K);
 * the block is forced to BF16 when it is strictly above rho.
 * ==================================================================== */

int64_t orc_outlier_count(const uint16_t *x, int64_t M, int64_t K, double kappa)
{
    const double kk = kappa * kappa;
    int64_t count = 0;
#pragma omp parallel for schedule(static) reduction(+ : count)
    for (int64_t m = 0; m < M; m++) {
        double S = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double v = (double)orc_bf16_value(x[m * K + k]);
            S += v * v;
        }
        const double rhs = kk * S;
        for (int64_t k = 0; k < K; k++) {
            double v = (double)orc_bf16_value(x[m * K + k]);
            if (v * v * (double)K > rhs)
                count++;
        }
    }
    return count;
}

/* The same count with the threshold moved by a relative band: lo counts the
 * elements above rhs*(1+rel), hi those above rhs*(1-rel).  A result whose row
 * sums were added in another order lies in [lo, hi]. */
void orc_outlier_count_band(const uint16_t *x, int64_t M, int64_t K, double kappa,
                            double rel, int64_t *lo, int64_t *hi)
{
    const double kk = kappa * kappa;
    int64_t clo = 0, chi = 0;
#pragma omp parallel for schedule(static) reduction(+ : clo, chi)
    for (int64_t m = 0; m < M; m++) {
        double S = 0.0;
        for (int64_t k = 0; k < K; k++) {
            double v = (double)orc_bf16_value(x[m * K + k]);
            S += v * v;
        }
        const double rhs = kk * S;
        for (int64_t k = 0; k < K; k++) {
            double v = (double)orc_bf16_value(x[m * K + k]);
            double t = v * v * (double)K;
            if (t > rhs * (1.0 + rel))
                clo++;
            if (t > rhs * (1.0 - rel))
                chi++;
        }
    }
    *lo = clo;
    *hi = chi;
}

int orc_pdr_force(int64_t count, int64_t n, double rho)
{
    if (n <= 0)
        return 0;
    return (double)count / (double)n > rho;
}

/* Full-precision linear of the BF16 route: y[m,n] = sum_k x[m,k] w[n,k] over
 * bf16 operands, products and sums in fp64; bound[m,n] = sum_k |x w|. */
int orc_gemm_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                  const int64_t *rows, int64_t n_rows, double *y, double *bound)
{
    if (M < 0 || N < 0 || K <= 0)
        return -1;
    const int64_t R = rows ? n_rows : M;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int64_t i = 0; i < R; i++) {
        int64_t m = rows ? rows[i] : i;
        if (m < 0 || m >= M) {
            err = 1;
            continue;
        }
        for (int64_t n = 0; n < N; n++) {
            double sum = 0.0, babs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double p = (double)orc_bf16_value(x[m * K + k]) *
                           (double)orc_bf16_value(w[n * K + k]);
                sum += p;
                babs += fabs(p);
            }
            if (y)
                y[i * N + n] = sum;
            if (bound)
                bound[i * N + n] = babs;
        }
    }
    return err ? -1 : 0;
}

/* ======================================================================
 * GELU of a DiT feed-forward layer, applied in the producing GEMM's
 * epilogue when the next layer's quantization prologue is fused there (the
 * pages ask the online Hadamard to add little overhead: [gist-en] §2.A
 * "Outlier Smoothing").  Exact erf form, GELU(x) = x Phi(x), in fp64 as
 * 0.5 x erfc(-x / sqrt 2), which does not cancel for negative x.
 * ==================================================================== */

double orc_gelu(double x)
{
    return 0.5 * x * erfc(-x / sqrt(2.0));
}
