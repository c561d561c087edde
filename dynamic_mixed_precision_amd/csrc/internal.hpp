// internal.hpp -- launchers shared between the translation units of libdmpq.
// Each launcher assumes its arguments were validated by the C-ABI layer
// (api.hip) and returns the hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dmpq {

// Workspace layout: per-workgroup partial results handed from the first
// kernel of a call to the second (partial fp64 sums, or partial float maxima
// for the NVFP4 amax).  Grids that use it are capped at kMaxPartials groups.
// Its contents need no initialization: every call writes before it reads.
constexpr int kMaxPartials = 2048;
constexpr int kMaxSums = 4;
constexpr size_t kWsBytes = sizeof(double) * kMaxSums * kMaxPartials;

struct Workspace {
    double *partial;  // kMaxSums * kMaxPartials doubles (also viewed as floats)
    explicit Workspace(void *ws) : partial(static_cast<double *>(ws)) {}
};

hipError_t launch_hq_int8(hipStream_t s, const uint16_t *x, int64_t M, int64_t K, int flags,
                          int8_t *q, float *s_row);
hipError_t launch_hq_nvfp4(hipStream_t s, const uint16_t *x, int64_t M, int64_t K, int flags,
                           uint8_t *codes, uint8_t *scales, float *g, const Workspace &ws);
// Partial maxima (floats) the first pass of launch_hq_nvfp4 writes without
// DMPQ_AMAX_GIVEN: one per workgroup, at most 1024 whatever the size.
int64_t hq_nvfp4_partials(int64_t M, int64_t K);
// Output tiles of the GEMMs (256 x 256 on every path that takes an epilogue):
// the number of per-tile maxima a fused-amax GEMM writes.
inline int64_t gemm_tiles(int64_t M, int64_t N) { return ((M + 255) / 256) * ((N + 255) / 256); }
hipError_t launch_w8_from_nvfp4(hipStream_t s, const uint8_t *cw, const uint8_t *sw,
                                const float *gw, int64_t N, int64_t K, int8_t *qw,
                                float *sw_row);
// launch_hq_int8 and launch_w8_from_nvfp4 (same K) in one launch
hipError_t launch_hq_int8_w8(hipStream_t s, const uint16_t *x, int64_t M, int64_t K, int flags,
                             int8_t *q, float *s_row, const uint8_t *cw, const uint8_t *sw,
                             const float *gw, int64_t N, int8_t *qw, float *sw_row);
// Row scales for the INT8 GEMM that converts an NVFP4 weight in its tile
// load: s_row = amax/127 and inv_row = 127/amax of each row of
// (E2M1 * E4M3) * gw, both 0 for a row whose reciprocal is not finite.
hipError_t launch_w8_row_scales(hipStream_t s, const uint8_t *cw, const uint8_t *sw, const float *gw,
                                int64_t N, int64_t K, float *s_row, float *inv_row);
bool hq_int8_supported(int64_t K);

hipError_t launch_gamma(hipStream_t s, const uint16_t *x_in, const uint16_t *x_out, int64_t n,
                        double *sums, const Workspace &ws);
hipError_t launch_tdc_skip(hipStream_t s, const uint16_t *x_in, const uint16_t *delta,
                           int64_t n, uint16_t *x_out);
hipError_t launch_tdc_refresh(hipStream_t s, const uint16_t *x_in, const uint16_t *x_out,
                              uint16_t *delta, int64_t n, int delta_valid, double *sums,
                              const Workspace &ws);

// Split of the last, partial wave of GEMM tiles along K.  A launch of T
// tiles on 256 CUs runs floor(T / 256) full waves and then a tail of T % 256
// tiles that leaves most CUs idle for a whole tile's time.  With a split plan
// the whole-tile kernel runs only the `full` tiles 0 .. full-1; a split
// kernel then runs tail * splits workgroups, each taking the K stages
// [s * nk / splits, (s + 1) * nk / splits) of one tail tile and storing its
// raw accumulators (kSplitWords words) in the split area; a fixup kernel adds
// each tail tile's partials in split order (deterministic) and runs the
// normal epilogue.  The split work is a kernel of its own so that the
// whole-tile kernel's register allocation is untouched.
struct SplitPlan {
    unsigned full;    // whole-tile workgroups (a multiple of 256), or every tile when splits == 1
    unsigned tail;    // tiles split along K
    unsigned splits;  // workgroups per tail tile (1: no split)
    int nk;           // K stages of a whole tile
};
constexpr size_t kSplitWords = 256 * 256;  // 32-bit words per split workgroup
constexpr unsigned kMaxSplitUnits = 256;   // split workgroups a launch may use
constexpr size_t kSplitAreaBytes = kMaxSplitUnits * kSplitWords * 4;
// Smallest K (elements) whose INT8 tail wave is split.  The INT8 tile is the
// shortest per K (the i8 MFMA has twice the fp16 rate): at K = 3072 its tail
// wave lasts about as long as the split's two extra launches and partial
// traffic (measured on the 17776-token shapes), so only longer K pay.  The
// NVFP4 and BF16 tails are split at every K.
constexpr int64_t kSplitMinKInt8 = 4096;
// Largest K of the GEMM entry points: the DMA kernels address 256 rows of an
// operand (at most 2 bytes per element) from a scalar base by 32-bit offsets.
constexpr int64_t kMaxGemmK = int64_t(1) << 22;

// epi: bit 0 GELU, bit 1 fused NVFP4 amax of the output into partial[tile]
// (bf16 output only); the GEMM tile is 256 x 256 on every path.  spart: the
// split area (kSplitAreaBytes), or NULL to run every tile whole.
hipError_t launch_gemm_int8(hipStream_t s, const int8_t *qa, const float *sa, const int8_t *qw,
                            const float *sw, int64_t M, int64_t N, int64_t K, int out_dtype,
                            void *y, int epi, float *partial, uint32_t *spart);
// The INT8 GEMM against an NVFP4 weight (cw, sw, gw) converted to INT8 in
// the weight-tile load with the row scales of launch_w8_row_scales; the
// same result as launch_gemm_int8 on the converted weight.  K % 128 == 0;
// whole tiles only (no split); epi and partial as in launch_gemm_int8.
hipError_t launch_gemm_int8_w4(hipStream_t s, const int8_t *qa, const float *sa, const uint8_t *cw,
                               const uint8_t *sw, const float *gw, const float *s_row,
                               const float *inv_row, int64_t M, int64_t N, int64_t K, int out_dtype,
                               void *y, int epi, float *partial);
hipError_t launch_gemm_bf16(hipStream_t s, const uint16_t *x, const uint16_t *w, int64_t M,
                            int64_t N, int64_t K, int out_dtype, void *y, int epi, float *partial,
                            uint32_t *spart);
// Fixup of a split launch with fp32 accumulators: y = (sum * gA) * gW (gA, gW
// read from device memory; NULL reads as 1).
hipError_t launch_f32_fixup(hipStream_t s, const float *ga, const float *gw, int64_t M, int64_t N,
                            void *y, unsigned tiles_m, unsigned tiles_n, unsigned group_m,
                            float *partial, const SplitPlan &sp, const uint32_t *spart,
                            int out_dtype, int epi);
hipError_t launch_outlier_count(hipStream_t s, const uint16_t *x, int64_t M, int64_t K,
                                double kappa, double *count, const Workspace &ws);
// Sum ns values per partial over nparts partials, in a fixed order, into out[ns].
hipError_t launch_finalize_sums(hipStream_t s, const double *partial, int nparts, int ns,
                                double *out);
hipError_t launch_gemm_nvfp4(hipStream_t s, const uint8_t *ca, const uint8_t *sa,
                             const float *ga, const uint8_t *cw, const uint8_t *sw,
                             const float *gw, int64_t M, int64_t N, int64_t K, int out_dtype,
                             void *y, int variant, int epi, float *partial, uint32_t *spart);

// Per-code (lowest, highest, count) of input bit patterns in [lo, hi) for the
// device converters (codec 0: E4M3 encoder; 1: hardware E2M1 converter).
hipError_t launch_codec_stats(hipStream_t s, int codec, uint32_t lo, uint32_t hi, uint32_t *stats);

// Grid for a grid-stride loop over `work` items with 256 threads per group.
inline unsigned stride_grid(int64_t work, int64_t per_group, unsigned cap) {
    int64_t g = (work + per_group - 1) / per_group;
    if (g < 1) g = 1;
    if (g > (int64_t)cap) g = cap;
    return (unsigned)g;
}

}  // namespace dmpq
