// device.hpp -- device helpers for the gfx950 kernels of libdmpq: bf16 bit
// conversions, the 16-point block Hadamard in registers, the E4M3 codec,
// wave reductions.  Compiled with -ffp-contract=off so every fp32
// expression below is a sequence of single IEEE round-to-nearest-even ops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dmpq {

constexpr int kWave = 64;

// ---- streaming 16-byte accesses (nontemporal: data touched once) ---------

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_nt16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_nt16(void *p, const uint4 &v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4 *>(p));
}

// ---- bf16 -----------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN -> canonical quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Same result as pack_bf16x2 for every non-NaN input, in one instruction
// (gfx950 v_cvt_pk_bf16_f32, round to nearest even; checked against
// f32_to_bf16 on all finite and infinite fp32 patterns).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    const v2bf r = __builtin_convertvector((v2f){lo, hi}, v2bf);
    return __builtin_bit_cast(uint32_t, r);
}

// Unpack 16 bf16 (two 16-byte words) into fp32.
__device__ __forceinline__ void unpack16(const uint4 &a, const uint4 &b, float v[16]) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; i++) {
        v[2 * i] = bf16_lo(w[i]);
        v[2 * i + 1] = bf16_hi(w[i]);
    }
}

// ---- 16-point Hadamard (Sylvester order), scaled by 1/4 --------------------
// Butterfly stages with spans 1, 2, 4, 8; pair (i, i+h) with (i & h) == 0
// becomes (a + b, a - b).  The 1/4 scaling is a power of two (exact for
// normal results).
__device__ __forceinline__ void fwht16(float v[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; i++) {
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] = v[i] * 0.25f;
}

// ---- E4M3 (OCP FN: bias 7, max 448, no inf) -------------------------------

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag = (e == 0) ? (float)m * 0.001953125f  // m * 2^-9
                         : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (c & 0x80u) ? -mag : mag;
}

// Non-negative v -> nearest E4M3 code, ties to even, saturating to 448; a NaN
// (Inf/Inf: a block holding an infinity of a tensor whose amax is infinite)
// encodes as 0, a zero scale.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float v) {
    if (!(v < 448.0f)) return v >= 448.0f ? 0x7Eu : 0u;
    if (v < 0.015625f) {                      // below 2^-6: subnormal grid m * 2^-9
        return (uint32_t)__builtin_rintf(v * 512.0f);  // 0..8 (8 = 2^-6, the first normal)
    }
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFFu + ((u >> 20) & 1u);         // RNE at mantissa bit 20
    uint32_t code = (u >> 20) - (120u << 3);  // rebias 127 -> 7, keep 3 mantissa bits
    return code > 0x7Eu ? 0x7Eu : code;
}

// ---- wave reductions --------------------------------------------------------

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, W));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) { return group_max<kWave>(v); }

}  // namespace dmpq
