// fp4_frag.h -- operand helpers shared by the gfx950 matrix-core kernels:
// vector types of the MFMA operands, raw buffer loads, and the exact
// NVFP4 -> f16 dequantization of an 8-element fragment.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsfp4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit dwords, range checked
// Cache-policy operand of a buffer load that marks it non-temporal (the nt bit
// of gfx950's sc0/nt/sc1 policy field): data read once, streamed past the caches.
constexpr int kStreamPolicy = 2;

// NVFP4 block-scale byte -> f16 holding S_b * 2^-8.  E4M3 (bias 7) and f16
// (bias 15) line up field by field: the E4M3 exponent and mantissa bits moved to
// f16's exponent and top mantissa bits give the same value times 2^-8,
// subnormals included (and every byte, the NaN pattern too, maps to a finite
// f16).  The 2^8 comes back through the conversion's power-of-two scale in
// dequant8, so e * S_b is formed exactly.
__device__ __forceinline__ _Float16 scale_h(uint32_t byte) {
    return __builtin_bit_cast(_Float16, (unsigned short)((byte & 0x7Fu) << 7));
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times the
// block scale -> eight exact f16.  The gfx950 scaled conversion applies only the
// exponent of its fp32 scale operand, so it is used for the exact factor 2^8 and
// the E4M3 scale (times 2^-8) is applied with a packed f16 multiply; every
// product e * S_b has at most 6 significant bits and lies in [2^-10, 2688], so
// both steps are exact.
__device__ __forceinline__ half8 dequant8(uint32_t w, _Float16 s) {
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0);
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1);
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2);
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
    const half2v s2 = {s, s};
    p0 *= s2; p1 *= s2; p2 *= s2; p3 *= s2;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Dword u of a 16-byte fragment.
__device__ __forceinline__ uint32_t word(const uint4& v, int u) {
    return u == 0 ? v.x : (u == 1 ? v.y : (u == 2 ? v.z : v.w));
}

// 16-byte raw buffer load (out-of-range offsets read zeros), with the given
// cache-policy bits.
template <int CPOL = 0>
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

}  // namespace rsfp4
