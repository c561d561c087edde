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

// ---- NVFP4 -> INT8 weight requantization ----------------------------------

// The 16 values (E2M1 value * E4M3 value) * g of one NVFP4 block in fp32:
// codes c (8 bytes, element 2i in the low nibble of byte i), block scale s
// (the decoded E4M3 value), tensor scale g.  The E2M1 values come from the
// hardware converter (v_cvt_scalef32_pk_f32_fp4 with scale 1.0: exact, low
// nibble first); E2M1 x E4M3 is exact in fp32, so only the product by g
// rounds.
__device__ __forceinline__ void nvfp4_block_values(const uint2 c, float s, float g, float v[16]) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    v2f e[8];  // the byte select is an immediate
    e[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 0);
    e[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 1);
    e[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 2);
    e[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.x, 1.0f, 3);
    e[4] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 0);
    e[5] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 1);
    e[6] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 2);
    e[7] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c.y, 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float lo = e[i].x, hi = e[i].y;  // scalars first: no element-lvalue casts
        v[2 * i] = (lo * s) * g;
        v[2 * i + 1] = (hi * s) * g;
    }
}

// Codes of one 16-block, q = RNE(v * inv) as bytes.  For |v| <= amax,
// |fl(v * inv)| < 127.5 (inv = fl(127/amax), two roundings of at most 2^-24
// each), so no clamp is needed; adding 1.5 * 2^23 rounds fl(v * inv) to an
// integer in the low mantissa bits (ties to even, as rint), whose low byte
// is the two's-complement code.  Every value of a row satisfies the bound,
// because amax is the row's maximum.  Non-finite values follow the library's
// rule: a NaN product (a NaN input, or an infinity times the zero reciprocal
// of a row whose amax is infinite) stays NaN through the add, keeping its
// payload, and it codes 0 when the payload's low byte is zero.  That holds
// for every NaN of a row that is not a zero row: bf16 data carries 16 zero
// low bits, and invalid operations make the default NaN.  (A NaN tensor
// scale of an NVFP4 weight makes every value of a row NaN, so the row is a
// zero row, which the caller stores as zeros.)  Two operations per value
// plus the byte packing.
__device__ __forceinline__ uint4 int8_codes_magic(const float v[16], float inv) {
    uint32_t t[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
        const float p = v[j] * inv;
        t[j] = __float_as_uint(p + 12582912.0f);
    }
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        // v_perm_b32: selector byte n picks byte n of {hi, lo} (0-3 lo, 4-7 hi)
        const uint32_t lo = __builtin_amdgcn_perm(t[4 * k + 1], t[4 * k], 0x0c0c0400u);
        const uint32_t hi = __builtin_amdgcn_perm(t[4 * k + 3], t[4 * k + 2], 0x0c0c0400u);
        w[k] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
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
