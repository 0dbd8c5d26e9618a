// codec.h -- device-side E2M1 / E4M3 / E8M0 codecs for the gfx950 kernels.
//
// Formats as defined on the ResServe page (arXiv 2611.08713), Section 2 and
// Figure 1: E2M1 elements (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), E4M3 block
// scales (largest finite 448) for NVFP4, power-of-two E8M0 block scales for
// MXFP4.  Every encoder rounds to nearest with ties to even and saturates; the
// arithmetic is IEEE binary32 (these files build with -ffp-contract=off and
// without fast-math, so division is correctly rounded and nothing fuses).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsfp4 {

// Magnitude code (0..7) of the E2M1 value nearest to u >= 0, ties to the even
// code, saturating at 6. The midpoints between neighbouring magnitudes are
// 0.25, 0.75, 1.25, 1.75, 2.5, 3.5 and 5; at a midpoint the even code wins, so
// the comparison is "<=" towards an even lower neighbour and "<" towards an
// odd one. A NaN argument compares false everywhere and gives code 0.
__device__ __forceinline__ uint32_t e2m1_mag(float u) {
    uint32_t c = 0;
    c += (u > 0.25f);
    c += (u >= 0.75f);
    c += (u > 1.25f);
    c += (u >= 1.75f);
    c += (u > 2.5f);
    c += (u >= 3.5f);
    c += (u > 5.0f);
    return c;
}

// Signed E2M1 value of a 4-bit code as float (bit 3 = sign).
__device__ __forceinline__ float e2m1_val(uint32_t code) {
    // magnitudes packed as halves of 2*value: 0,1,2,3,4,6,8,12
    const uint32_t twice = (0xC8643210u >> (4 * (code & 7u))) & 15u;
    float v = (float)twice * 0.5f;
    return (code & 8u) ? -v : v;
}

// E4M3 (FN variant) through gfx950's FP8 conversions (v_cvt_pk_fp8_f32 and
// v_cvt_f32_fp8), which use the OCP E4M3FN format on this chip.  Measured on
// the MI355X against the software rule (nearest finite value, ties to the even
// code, saturating at 448 = 0x7e): the encoder rounds to nearest even into the
// subnormals and agrees for every 0 < t <= 464 tried (all grid points, their
// midpoints and one ulp either side of each, 2^20 log-uniform values); above
// 464 it returns the NaN code 0x7f, so t is clamped to 448 first (every
// t >= 448 saturates to 448 anyway).  The decoder returns the exact value of
// every finite code.
//
// E4M3 byte -> value, for bytes 0x00..0x7e (non-negative scales).
__device__ __forceinline__ float e4m3_val(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// Non-negative t -> E4M3 byte: nearest finite value, ties to even code,
// saturating at 448 (0x7e, never the NaN code 0x7f); t NaN or <= 0 -> 0.
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
    const uint32_t code = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(t, 448.0f), 0.0f, 0, false) & 0xFFu;
    return t > 0.0f ? code : 0u;                                          // NaN and <= 0 -> 0
}

// gfx950 conversions between fp32 and E2M1 (v_cvt_scalef32_pk_fp4_f32 and
// v_cvt_scalef32_pk_f32_fp4).  Measured on the MI355X: the encoder divides by
// the power of two given by the scale operand's exponent field (the mantissa is
// ignored; a denormal scale acts as 2^-127) and rounds to nearest, ties to the
// even code, saturating at 6 (infinities too); the sign of zero and of inputs
// that round to zero is kept, and denormal inputs are not flushed.  So with a
// power-of-two scale X in [2^-127, 2^127] the code is exactly E2M1_RNE(v / X),
// the rule of e2m1_mag plus the input's sign bit.  The decoder returns the
// signed value times the scale's power of two.
//
// Codes of a and b into byte SEL of `old` (a in the low nibble).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float a, float b, float pow2_scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, pow2_scale, SEL);
}
// Signed values of the two codes in byte SEL of `packed`, times pow2_scale.
typedef float rsfp4_float2v __attribute__((ext_vector_type(2)));
template <int SEL>
__device__ __forceinline__ rsfp4_float2v e2m1_unpack2(uint32_t packed, float pow2_scale) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, pow2_scale, SEL);
}

// MXFP4: E8M0 byte for a block whose largest magnitude is a >= 0:
// floor(log2 a) - 2 biased by 127, clamped to [0, 254]; a == 0 -> 0.
__device__ __forceinline__ uint32_t e8m0_for_amax(float a) {
    const uint32_t bits = __float_as_uint(a);
    const int ef = (int)(bits >> 23);                         // a >= 0: no sign
    const int fl_sub = (31 - __builtin_clz(bits | 1u)) - 149;  // subnormal: leading one
    const int fl = ef > 0 ? ef - 127 : fl_sub;                 // floor(log2 a)
    int e = fl - 2;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    return a > 0.0f ? (uint32_t)(e + 127) : 0u;
}

// E8M0 byte -> 2^(b-127) as binary32 (b = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_val(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_rne(float v) {
    const uint32_t b = __float_as_uint(v);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x0040u);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Output store of the linear kernels: fp32, or bf16 rounded to nearest even.
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v, int bf16) {
    if (bf16)
        reinterpret_cast<uint16_t*>(y)[idx] = bf16_rne(v);
    else
        reinterpret_cast<float*>(y)[idx] = v;
}

}  // namespace rsfp4
