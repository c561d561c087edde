/*
 * oracle.h -- plain CPU reference ("oracle") for the dynamic mixed-precision
 * quantized linear layer of 6Bit-Diffusion (arXiv 2603.18742).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares source with it.
 *
 * Page citations use these short names (the pages are summaries of the paper):
 *   [gist-en]  gist.science/paper/2603.18742, English summary
 *   [gist-it]  gist.science/it/paper/2603.18742, Italian summary
 *   [gist-zh]  gist.science/zh/paper/2603.18742, Chinese explainer and
 *              technical summary ("technical" part unless noted)
 *   [abstract] chatpaper.ai page carrying the paper's English abstract
 *
 * Conventions: bf16 values travel as uint16_t bit patterns; E4M3 block scales
 * and packed E2M1 codes as uint8_t; tensors are row-major with K contiguous.
 * Every fp32 operation below is one IEEE round-to-nearest-even operation
 * (the file is compiled with -ffp-contract=off, no fast-math); reductions
 * accumulate in fp64.
 *
 * Parity unpinned (the pages fix no value or recipe for these, so the oracle
 * and the GPU agree with each other but nothing on the pages confirms them):
 *   - the NVFP4 two-level scale recipe (tensor scale maps the tensor amax to
 *     6*448, block scale = E4M3 of 448*amax_b/amax);
 *   - the NVFP4 -> INT8 weight conversion (per-output-channel absmax requant);
 *   - Gamma's base (L1 norm of the block input) and TDC "similarity" read as
 *     the relative L1 distance of the last two deltas;
 *   - alpha, beta, tau, eps_sim, delta_acc values (synthetic);
 *   - PDR's "outlier" (|x| above kappa times the token row's RMS) and its
 *     kappa and rho values.
 */
#ifndef DMPQ_ORACLE_H
#define DMPQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* flags for the quantizers: bit0 set = skip the block Hadamard (test hook) */
#define ORC_NO_HADAMARD 1

/* OpenMP threads the oracle's parallel loops use (for reporting). */
int orc_max_threads(void);
/* Threads for the oracle's later parallel loops (timing runs; n > 0). */
void orc_set_threads(int n);

/* ---- codecs ---------------------------------------------------------- */
uint16_t orc_bf16_round(float f);        /* fp32 -> bf16 bits, RNE; NaN -> 0x7FC0 */
float    orc_bf16_value(uint16_t b);     /* bf16 bits -> fp32 (exact) */
float    orc_e2m1_value(uint8_t code);   /* 4-bit code (low nibble) -> value */
uint8_t  orc_e2m1_encode(float v);       /* v -> nearest code, ties to even, saturating at 6; NaN -> 0 */
float    orc_e4m3_value(uint8_t code);   /* finite OCP E4M3 (FN) code -> value */
uint8_t  orc_e4m3_encode(float v);       /* v >= 0 -> nearest code, ties to even, saturating at 448; NaN -> 0 */

/* ---- block Hadamard -------------------------------------------------- */
void orc_fwht16(const float in[16], float out[16]);

/* ---- activation quantizers ------------------------------------------- */
int orc_quant_int8(const uint16_t *x, int64_t M, int64_t K, int flags,
                   int8_t *q, float *s_row);
int orc_quant_nvfp4(const uint16_t *x, int64_t M, int64_t K, int flags,
                    uint8_t *codes, uint8_t *scales, float *g);

/* ---- offline weight preparation -------------------------------------- */
#define ORC_W8_FROM_NVFP4 0
#define ORC_W8_DIRECT     1
int orc_prep_weight(const uint16_t *w, int64_t N, int64_t K, int int8_mode,
                    uint8_t *cw, uint8_t *sw, float *gw,
                    int8_t *qw, float *sw_row);
/* The FROM_NVFP4 step alone: INT8 weight from an NVFP4 weight (cw, sw, gw). */
int orc_w8_from_nvfp4(const uint8_t *cw, const uint8_t *sw, const float *gw,
                      int64_t N, int64_t K, int8_t *qw, float *sw_row);

/* ---- GEMMs (rows == NULL: all M rows; else the n_rows listed rows, and the
 *      outputs hold n_rows x N values in list order) -------------------- */
int orc_gemm_int8(const int8_t *qa, const float *sa, const int8_t *qw,
                  const float *sw, int64_t M, int64_t N, int64_t K,
                  const int64_t *rows, int64_t n_rows,
                  int32_t *acc, float *y);
int orc_gemm_nvfp4(const uint8_t *ca, const uint8_t *sa, float ga,
                   const uint8_t *cw, const uint8_t *sw, float gw,
                   int64_t M, int64_t N, int64_t K,
                   const int64_t *rows, int64_t n_rows,
                   double *y, double *bound);

/* ---- Gamma predictor and router -------------------------------------- */
void   orc_gamma_sums(const uint16_t *x_in, const uint16_t *x_out, int64_t n,
                      double sums[2]);
double orc_gamma(const double sums[2]);
#define ORC_ROUTE_NVFP4 0
#define ORC_ROUTE_INT8  1
void orc_route(const double *sums /* NULL = Gamma missing */, int n_lin,
               const double *alpha, const double *beta, double tau,
               double *gamma_out, double *err_out, uint8_t *route_out);

/* ---- Temporal Delta Cache -------------------------------------------- */
typedef struct {
    int64_t n_refresh;   /* completed refreshes (computed steps) */
    double  d;           /* relative L1 distance of the last two deltas */
    double  acc;         /* accumulated error over the current run of skips */
    int32_t delta_valid; /* a delta is cached */
    int32_t gamma_valid; /* gamma below holds the last computed step's Gamma */
    double  gamma;
} orc_tdc_state;

void orc_tdc_init(orc_tdc_state *st);
int  orc_tdc_decide(const orc_tdc_state *st, double eps_sim, double delta_acc);
void orc_tdc_skip(const uint16_t *x_in, const uint16_t *delta, int64_t n,
                  uint16_t *x_out);
void orc_tdc_refresh(const uint16_t *x_in, const uint16_t *x_out,
                     uint16_t *delta, int64_t n, int delta_valid,
                     double sums[4]);
void orc_tdc_commit_skip(orc_tdc_state *st);
void orc_tdc_commit_refresh(orc_tdc_state *st, const double sums[4]);

/* ---- Purified Delta Refresh and the BF16 route ---------------------- */
int64_t orc_outlier_count(const uint16_t *x, int64_t M, int64_t K, double kappa);
void orc_outlier_count_band(const uint16_t *x, int64_t M, int64_t K, double kappa,
                            double rel, int64_t *lo, int64_t *hi);
int orc_pdr_force(int64_t count, int64_t n, double rho);
int orc_gemm_bf16(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                  const int64_t *rows, int64_t n_rows, double *y, double *bound);

/* ---- GELU (fused producer epilogue) --------------------------------- */
double orc_gelu(double x);

#ifdef __cplusplus
}
#endif
#endif
