// selftest.hip -- exhaustive check of the device converters the quantizers
// use: the E4M3 block-scale encoder (e4m3_encode_nonneg) and the hardware
// E2M1 converter (v_cvt_scalef32_pk_fp4_f32, scale 1.0).  Not on the hot
// path: it exists so that tests can compare the converters with an
// independent encoder on every finite fp32 input.
//
// Both converters are monotone and piecewise constant in the input's bit
// pattern (for non-negative inputs; E2M1 negative inputs mirror them), so
// per output code the lowest and the highest input pattern that produce it
// and the number of patterns that do determine the converter completely:
// if they equal the reference's, every pattern agrees.
#include "device.hpp"
#include "internal.hpp"

namespace dmpq {

constexpr uint32_t kChunk = 4096;  // consecutive patterns per thread

__global__ __launch_bounds__(256) void codec_stats_init(uint32_t *stats, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        stats[3 * i] = 0xFFFFFFFFu;
        stats[3 * i + 1] = 0u;
        stats[3 * i + 2] = 0u;
    }
}

__device__ __forceinline__ void flush_run(uint32_t *stats, uint32_t code, uint32_t first, uint32_t last) {
    atomicMin(&stats[3 * code], first);
    atomicMax(&stats[3 * code + 1], last);
    atomicAdd(&stats[3 * code + 2], last - first + 1u);
}

// codec 0: E4M3 of the non-negative float with pattern p, codes 0..126.
// codec 1: E2M1 of +f and -f, codes 0..7 and 8..15 (stats rows 0..15).
// Patterns [lo, hi); each thread walks a contiguous chunk and flushes one
// run of equal codes at a time (a few atomics per chunk).
__global__ __launch_bounds__(256) void codec_stats_kernel(int codec, uint32_t lo, uint32_t hi,
                                                          uint32_t *stats) {
    const uint64_t c0 = (uint64_t)lo + ((uint64_t)blockIdx.x * 256 + threadIdx.x) * kChunk;
    if (c0 >= hi) return;
    const uint32_t first = (uint32_t)c0;
    const uint32_t last = (uint32_t)(c0 + kChunk < hi ? c0 + kChunk - 1 : hi - 1);
    if (codec == 0) {
        uint32_t run = first, cur = e4m3_encode_nonneg(__uint_as_float(first));
        for (uint32_t p = first + 1; p != last + 1; p++) {
            const uint32_t c = e4m3_encode_nonneg(__uint_as_float(p));
            if (c != cur) {
                flush_run(stats, cur, run, p - 1);
                run = p;
                cur = c;
            }
        }
        flush_run(stats, cur, run, last);
    } else {
        auto enc = [](uint32_t p) {
            const float v = __uint_as_float(p);
            // low nibble: E2M1(+v); high nibble: E2M1(-v)
            return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, -v, 1.0f, 0) & 0xFFu;
        };
        uint32_t run = first, cur = enc(first);
        for (uint32_t p = first + 1; p != last + 1; p++) {
            const uint32_t c = enc(p);
            if (c != cur) {
                flush_run(stats, cur & 15u, run, p - 1);
                flush_run(stats, cur >> 4, run, p - 1);
                run = p;
                cur = c;
            }
        }
        flush_run(stats, cur & 15u, run, last);
        flush_run(stats, cur >> 4, run, last);
    }
}

hipError_t launch_codec_stats(hipStream_t s, int codec, uint32_t lo, uint32_t hi, uint32_t *stats) {
    const int rows = codec == 0 ? 128 : 16;
    hipLaunchKernelGGL(codec_stats_init, dim3(1), dim3(256), 0, s, stats, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || hi <= lo) return e;
    const uint64_t threads = ((uint64_t)hi - lo + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(codec_stats_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, codec, lo,
                       hi, stats);
    return hipGetLastError();
}

}  // namespace dmpq
