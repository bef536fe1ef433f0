// kvq_device.h -- device-side building blocks shared by the libkvq kernels
// (gfx950 only): the OCP E4M3 codec on the native conversion instructions,
// vector types for MFMA operands, and wave-level helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef KVQ_CHECK
#define KVQ_CHECK 0   // 1: device-side checks of the caller's data contract (kvq_internal.h)
#endif

namespace kvq {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;   // OCP E4M3 largest finite magnitude
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bits_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bits_f32(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = f32_bits(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// ---- E4M3 encode: saturating round-to-nearest-even ---------------------
// The native v_cvt_pk_fp8_f32 rounds to nearest even; clamping to +-448 first
// makes overflow and Inf saturate instead of producing NaN.  NaN is mapped
// explicitly to 0x7F carrying the input's sign.  The clamp keeps -0.0, so a
// negative value that rounds to zero encodes as 0x80.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    float c = __builtin_fminf(__builtin_fmaxf(y, -kE4M3Max), kE4M3Max);
    uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
    if (__builtin_isnan(y)) code = 0x7Fu | ((f32_bits(y) >> 24) & 0x80u);
    return code;
}

// Encode 4 floats into one little-endian word of E4M3 codes.
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    return e4m3_encode(a) | (e4m3_encode(b) << 8) | (e4m3_encode(c) << 16) | (e4m3_encode(d) << 24);
}

// ---- E4M3 decode (exact) -------------------------------------------------
// Two codes from the low (hi = false) or high (hi = true) half of a word.
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_pk_f32_fp8(w, true) : __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
}
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
}

// 8 codes (two words) -> 8 halves / 8 bf16 (MFMA operand order = byte order)
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
    f16x2 a = e4m3x2_to_f16(w0, false), b = e4m3x2_to_f16(w0, true);
    f16x2 c = e4m3x2_to_f16(w1, false), d = e4m3x2_to_f16(w1, true);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    bf16x2 a = e4m3x2_to_bf16(w0, false), b = e4m3x2_to_bf16(w0, true);
    bf16x2 c = e4m3x2_to_bf16(w1, false), d = e4m3x2_to_bf16(w1, true);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ---- E2M1 (4-bit) codec ----------------------------------------------------
// Values of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (bit 3 = sign).  Encode:
// round to nearest, ties to the even code, saturate above 6 (Inf too), NaN ->
// 7 with its sign.  Each comparison is one rounding boundary; `>` at a tie
// rounds down to the even code below, `>=` rounds up to the even code above.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    const float a = __builtin_fabsf(y);
    const uint32_t s = (f32_bits(y) >> 28) & 0x8u;
    if (__builtin_isnan(y)) return 0x7u | s;
    const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return c | s;
}

// Two E2M1 codes (byte `SEL` of w, low nibble first) as exact f16 values.  The
// conversion's scale operand is applied as a power of two only (it is meant
// for power-of-two microscaling), so E4M3 block scales are applied separately
// with an f16 multiply: a 2-bit E2M1 significand times a 4-bit E4M3 scale has
// at most 6 significant bits and lies in [2^-10, 2688], exact in f16.
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2_to_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// 8 codes (one word, element order = nibble order) times one f16 scale.
__device__ __forceinline__ f16x8 e2m1x8_scaled_f16(uint32_t w, _Float16 scale) {
    const f16x2 s = {scale, scale};
    const f16x2 a = e2m1x2_to_f16<0>(w) * s, b = e2m1x2_to_f16<1>(w) * s;
    const f16x2 c = e2m1x2_to_f16<2>(w) * s, d = e2m1x2_to_f16<3>(w) * s;
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One NVFP4 block: 16 bf16 elements (two 16-byte words, element order) with
// the tensor's global scale -> 16 E2M1 codes (one per word of `codes`) and the
// E4M3 block-scale code.  bscale = E4M3(block amax / fp32(6 * gscale)),
// e = fp32(value(bscale) * gscale), codes E2M1(x / e) (all zero when e == 0);
// a NaN element makes the block scale NaN.  Shared by the cache write and the
// decode kernel's fused append, so both store the same bytes.
__device__ __forceinline__ void nvfp4_quantize_group(const u32x4& w0, const u32x4& w1, float gscale,
                                                     uint32_t* codes, uint32_t* bcode) {
#pragma clang fp contract(off)
    float xf[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        xf[2 * j] = bf16_lo(w0[j]);
        xf[2 * j + 1] = bf16_hi(w0[j]);
        xf[8 + 2 * j] = bf16_lo(w1[j]);
        xf[8 + 2 * j + 1] = bf16_hi(w1[j]);
    }
    float bamax = 0.f;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float a = __builtin_fabsf(xf[j]);
        nan |= __builtin_isnan(a);
        bamax = a > bamax ? a : bamax;
    }
    if (nan) bamax = __builtin_nanf("");
    const float top = 6.0f * gscale;
    *bcode = e4m3_encode(bamax / top);
    const float e = e4m3x2_to_f32(*bcode, false)[0] * gscale;
#pragma unroll
    for (int j = 0; j < 16; ++j) codes[j] = e == 0.0f ? 0u : e2m1_encode(xf[j] / e);
}

// ---- wave helpers ----------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int mask) {
    int lane = __lane_id();
    return bits_f32((uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, (int)f32_bits(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum of a value and the same value 16 (or 32) lanes away, on gfx950's
// v_permlane16_swap / v_permlane32_swap (plain VALU ops, no LDS round trip as
// with ds_bpermute).  A swap of a register with itself leaves each lane the
// pair {v[i], v[i ^ 16]} (or ^ 32) across its two results, in an order that
// depends on the lane; max and + are commutative, so every lane gets the
// same bits as from shfl_xor.
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(f32_bits(v), f32_bits(v), false, false);
    return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(f32_bits(v), f32_bits(v), false, false);
    return fmaxf(bits_f32(r[0]), bits_f32(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(f32_bits(v), f32_bits(v), false, false);
    return bits_f32(r[0]) + bits_f32(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(f32_bits(v), f32_bits(v), false, false);
    return bits_f32(r[0]) + bits_f32(r[1]);
}

#if KVQ_CHECK
// One flag word per translation unit (a static device variable; read on the
// host with hipMemcpyFromSymbol by that unit's check_flags_* function).
static __device__ unsigned g_check_flags;
__device__ __forceinline__ void check_fail(unsigned bit) { atomicOr(&g_check_flags, bit); }
#else
__device__ __forceinline__ void check_fail(unsigned) {}
#endif

}  // namespace kvq
