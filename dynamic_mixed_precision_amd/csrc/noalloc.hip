// noalloc.hip -- the NVFP4 activation quantizer for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): the same kernels as
// dmpq_hadamard_quant_nvfp4, with the per-workgroup partial maxima of the
// first pass in a static device array instead of a caller workspace.
//
// The array below is a device symbol.  In host code its name is only a
// host-side stand-in, not a device address, so it is never passed to a kernel
// or a copy: each device's address comes from hipGetSymbolAddress, taken once
// per device with that device current, and kept in g_scratch.
#include "dmpq.h"
#include "internal.hpp"

#include <mutex>

namespace dmpq {

// The array has the size of the caller workspace the checked entry point
// takes (64 KiB); the first pass writes one float per workgroup and its grid
// is capped at 512 workgroups (hq_nvfp4_partials), so it holds the partials
// of any tensor.  Every call on a device shares that device's copy, which
// keeps the last call's contents: the first pass writes every partial the
// second reads, so nothing needs clearing, but calls that overlap on one
// device (different streams) race.
constexpr size_t kScratchBytes = kWsBytes;
static __device__ __align__(256) double scratch[kScratchBytes / sizeof(double)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device, once known

// Address of the current device's copy of `scratch` (set-up on the first call
// on each device, under the lock).
hipError_t scratch_of_current_device(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

dmpq_status set_last_error(dmpq_status code, const char *fmt, ...);  // api.hip
dmpq_status check_hq_nvfp4_args(const char *fn, const uint16_t *x, int64_t M, int64_t K, int flags,
                                const uint8_t *codes, const uint8_t *scales, const float *d_g);  // api.hip
}  // namespace dmpq

using namespace dmpq;

extern "C" dmpq_status dmpq_hadamard_quant_nvfp4_noalloc(hipStream_t stream, const uint16_t *x,
                                                         int64_t M, int64_t K, int flags,
                                                         uint8_t *codes, uint8_t *scales,
                                                         float *d_g) {
    // every argument is checked before the first HIP call
    if (dmpq_status st = check_hq_nvfp4_args(__func__, x, M, K, flags, codes, scales, d_g)) return st;
    if (flags & DMPQ_AMAX_GIVEN)
        return set_last_error(DMPQ_ERR_UNSUPPORTED,
                              "%s: DMPQ_AMAX_GIVEN reads the producer GEMM's workspace; use "
                              "dmpq_hadamard_quant_nvfp4", __func__);
    const size_t need = (size_t)hq_nvfp4_partials(M, K) * sizeof(float);
    if (need > kScratchBytes)
        return set_last_error(DMPQ_ERR_WORKSPACE,
                              "%s: M = %lld, K = %lld needs %zu bytes of scratch, the static "
                              "array holds %zu", __func__, (long long)M, (long long)K, need,
                              kScratchBytes);
    void *ws = nullptr;
    const hipError_t e = scratch_of_current_device(&ws);
    if (e != hipSuccess)
        return set_last_error(DMPQ_ERR_HIP, "%s: scratch address: %s", __func__, hipGetErrorString(e));
    // the checked entry point launches on the scratch (kWsBytes, the
    // workspace size it requires)
    return dmpq_hadamard_quant_nvfp4(stream, x, M, K, flags, codes, scales, d_g, ws, kScratchBytes);
}
