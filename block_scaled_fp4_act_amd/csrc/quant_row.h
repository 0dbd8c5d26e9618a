// quant_row.h -- the per-row activation quantizer (NVFP4 and MXFP4, with the
// residue), shared by the quantize kernel and the linear that quantizes its
// own rows.  A row is quantized by a group of waves, eight elements per thread
// per chunk (as in the ResServe page's quantizer, Appendix B.2, Algorithm 1),
// with the row held in registers throughout so it is read from HBM once:
//   1. row amax -> tensor scale s_g = amax / 2688 (NVFP4; Appendix B.2, Eq. 8
//      with the maximum taken per row)
//   2. block amax over the adjacent lanes that share a block (DPP lane swaps),
//      then the block scale:
//      NVFP4 E4M3_RNE(blockmax / (6 s_g)), MXFP4 E8M0 (Section 2, Figure 1)
//   3. element codes E2M1_RNE(v / s~) (Eq. 10) with the gfx950 FP4 conversion
//      (NVFP4: on the IEEE quotient; MXFP4: straight from v with the power-of-
//      two scale), packed into one store per thread
//   4. residue r = v - fl(s~ e) kept in the same registers (Section 4.4: the
//      residue is formed in registers, no second read of x), e from the
//      hardware decoder
//   5. steps 1-3 again on r with its own row amax; the row goes to record M+m.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "codec.h"
#include "layout.h"

namespace rsfp4 {

namespace {

constexpr int kQMaxThreads = 1024;

// Lane exchanges through DPP (no LDS round trip): quad permutations for the
// lanes that share a block, row mirrors and lane reads for the wave maximum.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // reverse within 8 lanes
constexpr int kDppMirror = 0x140;     // reverse within 16 lanes

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppXor1>(v));
    v = fmaxf(v, dpp<kDppXor2>(v));
    v = fmaxf(v, dpp<kDppHalfMirror>(v));
    v = fmaxf(v, dpp<kDppMirror>(v));   // every lane: max of its 16-lane row
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Maximum of non-negative values over the waves w0 .. w0 + nw - 1 of the
// workgroup (a row's waves); every thread of the workgroup takes part in the
// barrier.  `red` holds one slot per wave; callers alternate between two such
// arrays so one barrier per reduction suffices (the next write goes to the
// other array).
__device__ __forceinline__ float group_max(float v, float* red, int w0, int nw) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) red[wid] = v;
    __syncthreads();
    float r = red[w0];
    for (int i = 1; i < nw; ++i) r = fmaxf(r, red[w0 + i]);
    return r;
}

template <typename T, int EPT>
__device__ __forceinline__ void load_chunk(const T* p, float* v);

template <>
__device__ __forceinline__ void load_chunk<float, 8>(const float* p, float* v) {
    const float4* q = reinterpret_cast<const float4*>(p);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
// bf16 -> fp32 is exact: the bf16 bits become the high half of the fp32 bits
template <>
__device__ __forceinline__ void load_chunk<__hip_bfloat16, 8>(const __hip_bfloat16* p, float* v) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j + 0] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
}

// The NVFP4 block-scale quotient bm / b, b = RN(6 s_g) shared by the row.
// FAST rows (tensor scale in [2^-80, 2^80], as for the element quotients
// below) divide once per row, y = RN(1/b), and per block apply Markstein's
// correction: q = RN(bm y), the remainder bm - b q (exact), RN(q + r y) =
// RN(bm / b).  b and y are normal there and the quotient is at most 448;
// quotients below 2^-22 (which encode to byte 0 however they round) aside,
// bm >= 2^-100, so q is faithful and the remainder is exact and normal.
struct BlockDiv {
    float b, y;
};

template <bool FAST>
__device__ __forceinline__ BlockDiv make_block_div(float s_g) {
    BlockDiv d;
    d.b = 6.0f * s_g;
    d.y = FAST ? 1.0f / d.b : 0.0f;
    return d;
}

// Block scale of a block whose largest magnitude is bm: the scale byte and the
// effective element scale s~ (NVFP4: E4M3_RNE(bm / (6 s_g)) and S_b * s_g;
// MXFP4: the E8M0 rule and its power of two).
template <int FMT, bool FAST>
__device__ __forceinline__ float block_scale(float bm, float s_g, const BlockDiv& bd, uint32_t& sbyte) {
    if (FMT == kNV) {
        float q;
        if (FAST) {
            const float q0 = bm * bd.y;
            q = __builtin_fmaf(__builtin_fmaf(-bd.b, q0, bm), bd.y, q0);
        } else {
            q = bm / bd.b;
        }
        sbyte = e4m3_encode(q);
        return e4m3_val(sbyte) * s_g;
    }
    sbyte = e8m0_for_amax(bm);
    return e8m0_val(sbyte);
}
template <int FMT>
__device__ __forceinline__ float block_scale(float bm, float s_g, uint32_t& sbyte) {
    return block_scale<FMT, false>(bm, s_g, make_block_div<false>(s_g), sbyte);
}

// Element codes with the hardware conversion (codec.h): MXFP4 converts v with
// the block's power-of-two scale directly; NVFP4 first forms the quotient
// v / s~ rounded to nearest and converts it with scale 1.  A zero s~ (zero
// block, or a block scale that rounds to 0) gives a zero of v's sign.  Dequantized values come back through the decoder: fl(s~ * e) for
// NVFP4 (the decoder's e is exact), X * e exactly for MXFP4.
// The NVFP4 element quotient v / s~, rounded to nearest.  A chunk's elements
// share s~, so the common case divides once per chunk: y = RN(1/s~) (an IEEE
// division), then per element q = RN(v y), the remainder r = v - s~ q (exact,
// one fma) and RN(q + r y) (one fma) -- Markstein's correction, which returns
// RN(v / s~) when y is the correctly rounded reciprocal and q a faithful
// quotient, with no under- or overflow on the way; the sign of zero is copied
// from v.  FAST is taken for rows whose tensor scale lies in [2^-80, 2^80]:
// then s~ and y are normal, |v / s~| stays below 7, and the remainders of
// quotients near the E2M1 rounding thresholds are normal.  Other rows divide.
// s~ = 0 (zero block) uses y = 0 with a unit divisor: every quotient is a
// zero of v's sign, as v / inf is.
struct Quot {
    float b, y, sd;
};

template <int FMT, bool FAST>
__device__ __forceinline__ Quot make_quot(float st) {
    Quot q;
    const bool z = st == 0.0f;
    q.b = z ? 1.0f : st;
    q.y = FAST ? (z ? 0.0f : 1.0f / st) : 0.0f;
    q.sd = z ? __builtin_inff() : st;
    return q;
}

template <bool FAST>
__device__ __forceinline__ float quot(float a, const Quot& d) {
    if (!FAST) return a / d.sd;
    const float q0 = a * d.y;
    const float r = __builtin_fmaf(-d.b, q0, a);
    return __builtin_copysignf(__builtin_fmaf(r, d.y, q0), a);
}

template <int FMT, int SEL, bool FAST>
__device__ __forceinline__ uint32_t enc2(uint32_t packed, float a, float b, float st, const Quot& d) {
    if (FMT == kNV) return e2m1_pack2<SEL>(packed, quot<FAST>(a, d), quot<FAST>(b, d), 1.0f);
    return e2m1_pack2<SEL>(packed, a, b, st);
}

// Rows whose NVFP4 tensor scale allows the one-division quotient.
__device__ __forceinline__ bool fast_quot_row(float s_g) {
    return s_g >= 8.271806125530277e-25f && s_g <= 1.2089258196146292e24f;   // 2^-80, 2^80
}

template <int FMT, int SEL>
__device__ __forceinline__ rsfp4_float2v dec2(uint32_t packed, float st) {
    if (FMT == kNV) {
        const rsfp4_float2v e = e2m1_unpack2<SEL>(packed, 1.0f);
        return rsfp4_float2v{st * e[0], st * e[1]};
    }
    return e2m1_unpack2<SEL>(packed, st);
}

// Encode EPT (4 or 8) values into packed nibbles (element e at bits 4e..4e+3)
// and replace them by their residues v - deq.
template <int FMT, int EPT, bool FAST>
__device__ __forceinline__ uint32_t encode_residue(float (&v)[EPT], float st) {
    const Quot dq = make_quot<FMT, FAST>(st);
    uint32_t packed = 0u;
    packed = enc2<FMT, 0, FAST>(packed, v[0], v[1], st, dq);
    packed = enc2<FMT, 1, FAST>(packed, v[2], v[3], st, dq);
    if (EPT == 8) {
        packed = enc2<FMT, 2, FAST>(packed, v[4], v[5], st, dq);
        packed = enc2<FMT, 3, FAST>(packed, v[6], v[7], st, dq);
    }
    rsfp4_float2v d;
    d = dec2<FMT, 0>(packed, st); v[0] -= d[0]; v[1] -= d[1];
    d = dec2<FMT, 1>(packed, st); v[2] -= d[0]; v[3] -= d[1];
    if (EPT == 8) {
        d = dec2<FMT, 2>(packed, st); v[4] -= d[0]; v[5] -= d[1];
        d = dec2<FMT, 3>(packed, st); v[6] -= d[0]; v[7] -= d[1];
    }
    return packed;
}

// ---- NVFP4 with a tensor scale given in advance (ResServe Appendix B.2) ----
// Eq. 8 bounds each 16-block by s_i = Max_i / 6; Eq. 9 stores s_i / alpha
// rounded to E4M3 and dequantizes with s~_i = alpha * S_i; Eq. 10 rounds the
// elements to E2M1 on that effective scale.  With alpha fixed (not derived
// from the row) the page's quantizer applies s~_i as a multiplier: codes of
// v * (1 / s~_i), reconstruction e / (1 / s~_i).  That reading is this
// operator's; the row-scaled quantizer above divides by s~ instead.
struct MulScale {
    uint32_t sbyte;   // the E4M3 byte S_i
    float mult;       // 1 / (alpha S_i), or 0 where alpha S_i is 0
};

__device__ __forceinline__ MulScale block_scale_alpha(float bm, float alpha) {
    MulScale m;
    m.sbyte = e4m3_encode((bm / 6.0f) / alpha);
    const float st = alpha * e4m3_val(m.sbyte);
    m.mult = st > 0.0f ? 1.0f / st : 0.0f;
    return m;
}

// E2M1 codes of the eight values v * mult, packed (element e at bits 4e);
// with RES, v becomes the residue v - e / mult (v itself where mult is 0).
template <bool RES>
__device__ __forceinline__ uint32_t encode_residue_mult(float (&v)[8], float mult) {
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = v[e] * mult;
    if (__builtin_expect(mult > 3.402823466e38f, 0)) {
        // the multiplier overflowed to infinity: a zero element would give
        // 0 * inf; its code is the zero of its sign, as for a finite multiplier
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = v[e] == 0.0f ? v[e] : u[e];
    }
    uint32_t packed = 0u;
    packed = e2m1_pack2<0>(packed, u[0], u[1], 1.0f);
    packed = e2m1_pack2<1>(packed, u[2], u[3], 1.0f);
    packed = e2m1_pack2<2>(packed, u[4], u[5], 1.0f);
    packed = e2m1_pack2<3>(packed, u[6], u[7], 1.0f);
    if (RES) {
        rsfp4_float2v d[4];
        d[0] = e2m1_unpack2<0>(packed, 1.0f);
        d[1] = e2m1_unpack2<1>(packed, 1.0f);
        d[2] = e2m1_unpack2<2>(packed, 1.0f);
        d[3] = e2m1_unpack2<3>(packed, 1.0f);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] - (mult > 0.0f ? d[e >> 1][e & 1] / mult : 0.0f);
    }
    return packed;
}

// Record header: the row's fp32 tensor scale (0 for MXFP4) and zero padding.
__device__ __forceinline__ void store_head(uint8_t* rec, float s_g, int lt) {
    if (lt == 0) *reinterpret_cast<uint4*>(rec) = make_uint4(__float_as_uint(s_g), 0u, 0u, 0u);
}

// Quantize the NC chunks of EPT elements held in v[] (in place: v becomes the
// residue): chunk j's codes go to codes[j * EPT / 2 ..], its block scale byte
// to scales[j / lanes-per-block].  s_g is the row's tensor scale (NVFP4);
// nchunks = K / EPT; the row's nt threads (a multiple of 64) hold chunks
// lt, lt + nt, ...  Only chunks of the part [j0, j0 + cw) are written (j0 and
// cw multiples of 64, so a wave's 64 chunks of one c are all in or all out);
// the others are quantized (for their residue) when all is set and skipped
// otherwise.
template <int FMT, int NC, int EPT, bool FAST>
__device__ __forceinline__ void quantize_chunks_q(float (&v)[NC][EPT], int nchunks, float s_g,
                                                  uint8_t* codes, uint8_t* scales, int lt, int nt, int j0, int cw,
                                                  bool all) {
    constexpr int LPB = (FMT == kNV ? 16 : 32) / EPT;   // lanes sharing one block
    const BlockDiv bd = make_block_div<FAST>(s_g);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = lt + nt * c;                   // chunk index
        const int jw = (lt & ~63) + nt * c;          // the wave's first chunk of this c
        const bool in = jw >= j0 && jw - j0 < cw;    // wave-uniform
        if (!in && !all) continue;
        float bm = 0.0f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) bm = fmaxf(bm, fabsf(v[c][e]));
        // the block's chunks sit in adjacent lanes of one wave (nt % 64 == 0)
        if (LPB >= 2) bm = fmaxf(bm, dpp<kDppXor1>(bm));
        if (LPB >= 4) bm = fmaxf(bm, dpp<kDppXor2>(bm));
        if (LPB >= 8) bm = fmaxf(bm, dpp<kDppHalfMirror>(bm));
        uint32_t sbyte;
        const float st = block_scale<FMT, FAST>(bm, s_g, bd, sbyte);   // effective element scale
        // codes, and v becomes the residue x - fl(s~ e) (exact: Sterbenz)
        const uint32_t packed = encode_residue<FMT, EPT, FAST>(v[c], st);
        if (in && j < nchunks) {
            if (EPT == 8)
                *reinterpret_cast<uint32_t*>(codes + 4 * (int64_t)j) = packed;
            else
                *reinterpret_cast<uint16_t*>(codes + 2 * (int64_t)j) = (uint16_t)packed;
            if ((j & (LPB - 1)) == 0) scales[j / LPB] = (uint8_t)sbyte;
        }
    }
}

// The row's quotient path is chosen once per row (the tensor scale is the same
// in every thread of the workgroup, so the branch does not diverge).
template <int FMT, int NC, int EPT>
__device__ __forceinline__ void quantize_chunks(float (&v)[NC][EPT], int nchunks, float s_g,
                                                uint8_t* codes, uint8_t* scales, int lt, int nt, int j0 = 0,
                                                int cw = 0x7fffffff, bool all = true) {
    if (FMT == kNV && !fast_quot_row(s_g))
        quantize_chunks_q<FMT, NC, EPT, false>(v, nchunks, s_g, codes, scales, lt, nt, j0, cw, all);
    else
        quantize_chunks_q<FMT, NC, EPT, true>(v, nchunks, s_g, codes, scales, lt, nt, j0, cw, all);
}

// One row, in two phases so a caller can issue other loads in between:
// row_load reads the row's chunks (zeros past K) into registers, row_quantize
// then runs steps 1-5 on them and writes the row's record (and, with_res, the
// residue's record).  The row's nt threads are lt = 0 .. nt - 1, waves w0 ..
// w0 + nt / 64 - 1 of the workgroup; every thread of the workgroup calls
// row_quantize (it holds two barriers), threads of no row with active = false.
// A row may be shared by several workgroups, each writing the part of chunks
// [j0, j0 + cw) (the heads with the part at j0 = 0): each forms both row
// maxima over the whole row (the residue's needs every base code), but only
// its part's residue codes.
template <int NC, int EPT, typename TIn>
__device__ __forceinline__ void row_load(const TIn* __restrict__ xr, int64_t K, int lt, int nt, bool active,
                                         float (&v)[NC][EPT]) {
    const int nchunks = (int)(K / EPT);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = lt + nt * c;
        if (active && j < nchunks) {
            load_chunk<TIn, EPT>(xr + EPT * (int64_t)j, v[c]);
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e) v[c][e] = 0.0f;
        }
    }
}

template <int FMT, int NC, int EPT>
__device__ __forceinline__ void row_quantize(float (&v)[NC][EPT], int64_t K, int lt, int nt, bool active, int with_res,
                                             uint8_t* rec, uint8_t* rrec, float (*red)[kQMaxThreads / 64],
                                             int j0 = 0, int cw = 0x7fffffff) {
    const int nchunks = (int)(K / EPT);
    const int w0 = (threadIdx.x - lt) >> 6, nw = nt >> 6;
    float tmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < EPT; ++e) tmax = fmaxf(tmax, fabsf(v[c][e]));
    const float amax = group_max(tmax, red[0], w0, nw);
    const float s_g = FMT == kNV ? amax / 2688.0f : 0.0f;
    if (active) {
        if (j0 == 0) store_head(rec, s_g, lt);
        quantize_chunks<FMT, NC, EPT>(v, nchunks, s_g, rec + kActHead, rec + kActHead + K / 2, lt, nt, j0, cw,
                                      with_res != 0);
    }
    if (!with_res) return;
    // v now holds the residue (zero in chunks past K): second row statistic.
    float rmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < EPT; ++e) rmax = fmaxf(rmax, fabsf(v[c][e]));
    const float ramax = group_max(rmax, red[1], w0, nw);
    const float r_g = FMT == kNV ? ramax / 2688.0f : 0.0f;
    if (active) {
        if (j0 == 0) store_head(rrec, r_g, lt);
        quantize_chunks<FMT, NC, EPT>(v, nchunks, r_g, rrec + kActHead, rrec + kActHead + K / 2, lt, nt, j0, cw,
                                      false);
    }
}

}  // namespace

}  // namespace rsfp4
