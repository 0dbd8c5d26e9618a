// quant.hip -- activation quantize + residue kernels (NVFP4 and MXFP4): the
// per-row dynamic-scale quantizer (one workgroup per row or, NVFP4 with few
// rows, per part of a row; T = 64..1024 threads; the row routine and its
// steps are in quant_row.h), the selective
// (K-Ext) quantizer and the given-tensor-scale quantizer of the page's
// Algorithm 1.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "codec.h"
#include "kernels.h"
#include "layout.h"
#include "quant_row.h"

namespace rsfp4 {

namespace {

// Row m is shared by `parts` workgroups (m = block / parts), the p-th writing
// chunks [p cw, (p + 1) cw) of both records.
template <int FMT, int NC, int EPT, typename TIn>
__global__ __launch_bounds__(kQMaxThreads) void quant_act_kernel(const TIn* __restrict__ x, int M,
                                                                 int64_t K, int with_res,
                                                                 uint8_t* __restrict__ act,
                                                                 int64_t row_bytes, int parts, int cw) {
    __shared__ float red[2][kQMaxThreads / 64];
    const int m = blockIdx.x / parts, p = blockIdx.x - m * parts;
    float v[NC][EPT];
    row_load<NC, EPT, TIn>(x + (int64_t)m * K, K, threadIdx.x, blockDim.x, true, v);
    row_quantize<FMT, NC, EPT>(v, K, threadIdx.x, blockDim.x, true, with_res, act + (int64_t)m * row_bytes,
                               act + (int64_t)(M + m) * row_bytes, red, p * cw, cw);
}

// Parts per row (NVFP4): with few rows a row's quantization is bound by one
// compute unit's VALU issue (the exact quotients), so rows of at least 512
// chunks (4096 elements) are shared by up to 8 workgroups, parts of a
// multiple of 64 chunks (whole waves) and at least 256 (four waves, one per
// SIMD), while rows x parts stay within the compute units.  Each part
// recomputes the row statistics; the residue's codes, half the work, split
// across the parts (the plain quantizer's codes entirely).  Measured in the
// compensated step at M = 8: K = 14336 18.0 against 18.7 us, K = 8192 30.8
// against 30.9-31.0 us, K = 4096 unchanged; MXFP4 (no divisions) is 0.2 us
// slower shared and keeps one workgroup per row.
void quant_parts(int M, int64_t nchunks, int num_cus, int* parts, int* cw) {
    int W = (int)(nchunks / 256);
    if (W > 8) W = 8;
    while (W > 1 && (int64_t)M * W > num_cus) --W;
    if (W < 1) W = 1;
    const int64_t per = ((nchunks + W - 1) / W + 63) / 64 * 64;
    *cw = (int)per;
    *parts = (int)((nchunks + per - 1) / per);
}

template <int FMT, int NC, int EPT, typename TIn>
hipError_t launch_quant_t(const void* x, int M, int64_t K, int with_res, void* act, int threads, int num_cus,
                          hipStream_t s) {
    const int64_t rb = act_row_bytes(FMT, K);
    int parts = 1, cw = 0x7fffffff;
    if (FMT == kNV && num_cus > 0) quant_parts(M, K / EPT, num_cus, &parts, &cw);
    hipLaunchKernelGGL((quant_act_kernel<FMT, NC, EPT, TIn>), dim3((unsigned)M * (unsigned)parts), dim3(threads), 0,
                       s, static_cast<const TIn*>(x), M, K, with_res, static_cast<uint8_t*>(act), rb, parts, cw);
    return hipGetLastError();
}

// Eight elements per thread (a row of up to 8192 in one chunk per thread, up to
// 1024 threads), NC chunks per thread for longer rows.  Eight rather than four
// elements per thread halves the threads that repeat a block's scale
// computation; with one row per compute unit the quantizer is bound by that
// unit's VALU issue, and at K = 4096 this measured 3.7 us against 4.4 us.
template <int FMT, typename TIn>
hipError_t launch_quant_f(const void* x, int M, int64_t K, int with_res, void* act, int num_cus, hipStream_t s) {
    const int64_t nch = K / 8;
    if (nch <= kQMaxThreads) {
        const int threads = (int)((nch + 63) / 64 * 64);
        return launch_quant_t<FMT, 1, 8, TIn>(x, M, K, with_res, act, threads, num_cus, s);
    }
    if (nch <= 2 * kQMaxThreads)
        return launch_quant_t<FMT, 2, 8, TIn>(x, M, K, with_res, act, kQMaxThreads, num_cus, s);
    return launch_quant_t<FMT, 4, 8, TIn>(x, M, K, with_res, act, kQMaxThreads, num_cus, s);
}

// ---------------------------------------------------------------- K-Ext --
// Selective compensation (ResServe Section 5.3, Eq. 6; Appendix B.1 and
// Algorithm 1): the record of row m holds K_eff = K + (K/8) k elements, the base
// codes of all K channels followed by the extension, the residues of the k
// channels that mask byte g selects in group g, in increasing channel order,
// group after group.  One thread owns one 8-channel group (EPT = 8), so its k
// extension elements are the contiguous run [g k, g k + k); an extension block
// (16 or 32 elements) spans blk / k adjacent lanes.  Residue blocks take the
// base row's tensor scale (the algorithm feeds one alpha to both block-scale
// steps), MXFP4 the E8M0 rule.

__device__ __forceinline__ uint32_t dpp_xor1_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xF, 0xF, false);
}

// Maximum over aligned runs of L adjacent lanes (L a power of two <= 32).
template <int L>
__device__ __forceinline__ float run_max(float bm) {
    if (L >= 2) bm = fmaxf(bm, dpp<kDppXor1>(bm));
    if (L >= 4) bm = fmaxf(bm, dpp<kDppXor2>(bm));
    if (L >= 8) bm = fmaxf(bm, dpp<kDppHalfMirror>(bm));
    if (L >= 16) bm = fmaxf(bm, dpp<kDppMirror>(bm));
    if (L >= 32) bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    return bm;
}

template <int FMT, int NC, int KS, typename TIn>
__global__ __launch_bounds__(kQMaxThreads) void quant_kext_kernel(const TIn* __restrict__ x, int64_t K,
                                                                  const uint8_t* __restrict__ masks,
                                                                  uint8_t* __restrict__ act,
                                                                  int64_t row_bytes) {
    constexpr int BLK = FMT == kNV ? 16 : 32;
    constexpr int LPE = BLK / KS;                 // lanes per extension block
    __shared__ float red[kQMaxThreads / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nchunks = (int)(K / 8);
    const TIn* xr = x + (int64_t)m * K;

    float v[NC][8];
    uint32_t mk[NC];
    float tmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = tid + (int)blockDim.x * c;
        if (j < nchunks) {
            load_chunk<TIn, 8>(xr + 8 * (int64_t)j, v[c]);
            mk[c] = masks[j];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = 0.0f;
            mk[c] = 0u;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, fabsf(v[c][e]));
    }
    const float amax = group_max(tmax, red, 0, blockDim.x >> 6);
    const int64_t KE = K + (K / 8) * KS;
    uint8_t* rec = act + (int64_t)m * row_bytes;
    uint8_t* codes = rec + kActHead;
    uint8_t* scales = codes + KE / 2;
    const float s_g = FMT == kNV ? amax / 2688.0f : 0.0f;
    store_head(rec, s_g, threadIdx.x);
    quantize_chunks<FMT, NC, 8>(v, nchunks, s_g, codes, scales, threadIdx.x, blockDim.x);   // v: residue from here on

    uint8_t* ecodes = codes + K / 2;
    uint8_t* escales = scales + K / BLK;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = tid + (int)blockDim.x * c;
        // the k selected residues of this group, lowest channel first
        float rs[KS];
        uint32_t rest = mk[c];
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            if (KS == 8) {
                rs[q] = v[c][q];
            } else {
                // lowest set bit still pending (a byte with fewer than k bits
                // falls back to channel 7: defined, in-register, no memory access)
                const int idx = rest ? __builtin_ctz(rest) : 7;
                float r = v[c][0];
#pragma unroll
                for (int e = 1; e < 8; ++e) r = idx == e ? v[c][e] : r;
                rs[q] = r;
                rest &= rest - 1u;
            }
        }
        float bm = 0.0f;
#pragma unroll
        for (int q = 0; q < KS; ++q) bm = fmaxf(bm, fabsf(rs[q]));
        bm = run_max<LPE>(bm);
        uint32_t sbyte;
        const float st = block_scale<FMT>(bm, s_g, sbyte);
        const Quot dq = make_quot<FMT, false>(st);       // the extension divides
        uint32_t packed = 0u;
        if (KS == 1) {
            packed = enc2<FMT, 0, false>(0u, rs[0], 0.0f, st, dq) & 15u;
        } else {
            packed = enc2<FMT, 0, false>(packed, rs[0], rs[KS > 1 ? 1 : 0], st, dq);
            if (KS >= 4) packed = enc2<FMT, 1, false>(packed, rs[KS >= 4 ? 2 : 0], rs[KS >= 4 ? 3 : 0], st, dq);
            if (KS == 8) {
                packed = enc2<FMT, 2, false>(packed, rs[KS == 8 ? 4 : 0], rs[KS == 8 ? 5 : 0], st, dq);
                packed = enc2<FMT, 3, false>(packed, rs[KS == 8 ? 6 : 0], rs[KS == 8 ? 7 : 0], st, dq);
            }
        }
        uint32_t pair = 0u;
        if (KS == 1) pair = packed | (dpp_xor1_u32(packed) << 4);   // even lane: its nibble low
        if (j < nchunks) {
            if (KS == 8) *reinterpret_cast<uint32_t*>(ecodes + 4 * (int64_t)j) = packed;
            if (KS == 4) *reinterpret_cast<uint16_t*>(ecodes + 2 * (int64_t)j) = (uint16_t)packed;
            if (KS == 2) ecodes[j] = (uint8_t)packed;
            if (KS == 1 && (j & 1) == 0) ecodes[j >> 1] = (uint8_t)pair;
            if ((j & (LPE - 1)) == 0) escales[j / LPE] = (uint8_t)sbyte;
        }
    }
}

template <int FMT, int NC, int KS, typename TIn>
hipError_t launch_kext_t(const void* x, int M, int64_t K, const uint8_t* masks, void* act, hipStream_t s) {
    const int64_t rb = act_row_bytes(FMT, K + (K / 8) * KS);
    const int64_t nch = K / 8;
    const int threads = nch >= kQMaxThreads ? kQMaxThreads : (int)((nch + 63) / 64 * 64);
    hipLaunchKernelGGL((quant_kext_kernel<FMT, NC, KS, TIn>), dim3(M), dim3(threads), 0, s,
                       static_cast<const TIn*>(x), K, masks, static_cast<uint8_t*>(act), rb);
    return hipGetLastError();
}

template <int FMT, int KS, typename TIn>
hipError_t launch_kext_nc(const void* x, int M, int64_t K, const uint8_t* masks, void* act, hipStream_t s) {
    const int64_t nch = K / 8;
    if (nch <= kQMaxThreads) return launch_kext_t<FMT, 1, KS, TIn>(x, M, K, masks, act, s);
    if (nch <= 2 * kQMaxThreads) return launch_kext_t<FMT, 2, KS, TIn>(x, M, K, masks, act, s);
    return launch_kext_t<FMT, 4, KS, TIn>(x, M, K, masks, act, s);
}

template <int FMT, typename TIn>
hipError_t launch_kext_f(const void* x, int M, int64_t K, const uint8_t* masks, int k, void* act,
                         hipStream_t s) {
    switch (k) {
        case 1: return launch_kext_nc<FMT, 1, TIn>(x, M, K, masks, act, s);
        case 2: return launch_kext_nc<FMT, 2, TIn>(x, M, K, masks, act, s);
        case 4: return launch_kext_nc<FMT, 4, TIn>(x, M, K, masks, act, s);
        default: return launch_kext_nc<FMT, 8, TIn>(x, M, K, masks, act, s);
    }
}

// ------------------------------------------------- paper numerics (alpha) --
// NVFP4 with one tensor scale alpha for the whole activation tensor (Appendix
// B.2, Eqs. 8-10), read from device memory (static or calibrated;
// rsfp4_nvfp4_tensor_alpha derives it from the data) and shared by x and r, so
// no row reduction runs: per 16-block the scale and multiplier of
// block_scale_alpha and the codes of encode_residue_mult.  Eight elements per
// thread, so a block's maximum spans two adjacent lanes.

template <int NC, bool RES>
__device__ __forceinline__ void quantize_chunks_alpha(float (&v)[NC][8], int nchunks, float alpha, uint8_t* codes,
                                                      uint8_t* scales) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = (int)threadIdx.x + (int)blockDim.x * c;
        float bm = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) bm = fmaxf(bm, fabsf(v[c][e]));
        bm = fmaxf(bm, dpp<kDppXor1>(bm));
        const MulScale ms = block_scale_alpha(bm, alpha);
        const uint32_t packed = encode_residue_mult<RES>(v[c], ms.mult);
        if (j < nchunks) {
            *reinterpret_cast<uint32_t*>(codes + 4 * (int64_t)j) = packed;
            if ((j & 1) == 0) scales[j >> 1] = (uint8_t)ms.sbyte;
        }
    }
}

template <int NC, typename TIn>
__global__ __launch_bounds__(kQMaxThreads) void quant_alpha_kernel(const TIn* __restrict__ x, int M, int64_t K,
                                                                   const float* __restrict__ alpha_p,
                                                                   int with_res, uint8_t* __restrict__ act,
                                                                   int64_t row_bytes) {
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nchunks = (int)(K / 8);
    const TIn* xr = x + (int64_t)m * K;
    const float alpha = *alpha_p;
    float v[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = tid + (int)blockDim.x * c;
        if (j < nchunks) {
            load_chunk<TIn, 8>(xr + 8 * (int64_t)j, v[c]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[c][e] = 0.0f;
        }
    }
    uint8_t* rec = act + (int64_t)m * row_bytes;
    store_head(rec, alpha, threadIdx.x);
    if (!with_res) {
        quantize_chunks_alpha<NC, false>(v, nchunks, alpha, rec + kActHead, rec + kActHead + K / 2);
        return;
    }
    quantize_chunks_alpha<NC, true>(v, nchunks, alpha, rec + kActHead, rec + kActHead + K / 2);
    uint8_t* rrec = act + (int64_t)(M + m) * row_bytes;
    store_head(rrec, alpha, threadIdx.x);
    quantize_chunks_alpha<NC, false>(v, nchunks, alpha, rrec + kActHead, rrec + kActHead + K / 2);
}

template <int NC, typename TIn>
hipError_t launch_alpha_t(const void* x, int M, int64_t K, const float* alpha, int with_res, void* act,
                          hipStream_t s) {
    const int64_t rb = act_row_bytes(kNV, K);
    const int64_t nch = K / 8;
    const int threads = nch >= kQMaxThreads ? kQMaxThreads : (int)((nch + 63) / 64 * 64);
    hipLaunchKernelGGL((quant_alpha_kernel<NC, TIn>), dim3(M), dim3(threads), 0, s,
                       static_cast<const TIn*>(x), M, K, alpha, with_res, static_cast<uint8_t*>(act), rb);
    return hipGetLastError();
}

template <typename TIn>
hipError_t launch_alpha_f(const void* x, int M, int64_t K, const float* alpha, int with_res, void* act,
                          hipStream_t s) {
    const int64_t nch = K / 8;
    if (nch <= kQMaxThreads) return launch_alpha_t<1, TIn>(x, M, K, alpha, with_res, act, s);
    if (nch <= 2 * kQMaxThreads) return launch_alpha_t<2, TIn>(x, M, K, alpha, with_res, act, s);
    return launch_alpha_t<4, TIn>(x, M, K, alpha, with_res, act, s);
}

// alpha = fl(fl(amax / 6) / 448) over n elements: clear, reduce the maximum
// (atomicMax on the binary32 bits, which order like the values for x >= 0),
// then finish in one thread.
__global__ void alpha_clear_kernel(float* alpha) { *reinterpret_cast<uint32_t*>(alpha) = 0u; }

template <typename TIn>
__global__ __launch_bounds__(256) void alpha_amax_kernel(const TIn* __restrict__ x, int64_t n, float* alpha) {
    float m = 0.0f;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        float v;
        if (sizeof(TIn) == 2)
            v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(x)[i] << 16);
        else
            v = reinterpret_cast<const float*>(x)[i];
        m = fmaxf(m, fabsf(v));
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) atomicMax(reinterpret_cast<uint32_t*>(alpha), __float_as_uint(m));
}

__global__ void alpha_finish_kernel(float* alpha) {
    const float amax = *alpha;
    *alpha = (amax / 6.0f) / 448.0f;
}

}  // namespace

hipError_t launch_quantize_act(int fmt, int xt_bf16, const void* x, int M, int64_t K, int with_res,
                               void* act, int num_cus, hipStream_t s) {
    if (fmt == kNV) {
        return xt_bf16 ? launch_quant_f<kNV, __hip_bfloat16>(x, M, K, with_res, act, num_cus, s)
                       : launch_quant_f<kNV, float>(x, M, K, with_res, act, num_cus, s);
    }
    return xt_bf16 ? launch_quant_f<kMX, __hip_bfloat16>(x, M, K, with_res, act, num_cus, s)
                   : launch_quant_f<kMX, float>(x, M, K, with_res, act, num_cus, s);
}

hipError_t launch_quantize_act_kext(int fmt, int xt_bf16, const void* x, int M, int64_t K,
                                    const uint8_t* masks, int k, void* act, hipStream_t s) {
    if (fmt == kNV)
        return xt_bf16 ? launch_kext_f<kNV, __hip_bfloat16>(x, M, K, masks, k, act, s)
                       : launch_kext_f<kNV, float>(x, M, K, masks, k, act, s);
    return xt_bf16 ? launch_kext_f<kMX, __hip_bfloat16>(x, M, K, masks, k, act, s)
                   : launch_kext_f<kMX, float>(x, M, K, masks, k, act, s);
}

hipError_t launch_quantize_act_alpha(int xt_bf16, const void* x, int M, int64_t K, const float* alpha,
                                     int with_res, void* act, hipStream_t s) {
    return xt_bf16 ? launch_alpha_f<__hip_bfloat16>(x, M, K, alpha, with_res, act, s)
                   : launch_alpha_f<float>(x, M, K, alpha, with_res, act, s);
}

hipError_t launch_tensor_alpha(int xt_bf16, const void* x, int64_t n, float* alpha, hipStream_t s) {
    hipLaunchKernelGGL(alpha_clear_kernel, dim3(1), dim3(1), 0, s, alpha);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (xt_bf16)
        hipLaunchKernelGGL(alpha_amax_kernel<__hip_bfloat16>, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const __hip_bfloat16*>(x), n, alpha);
    else
        hipLaunchKernelGGL(alpha_amax_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const float*>(x), n, alpha);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(alpha_finish_kernel, dim3(1), dim3(1), 0, s, alpha);
    return hipGetLastError();
}

}  // namespace rsfp4
