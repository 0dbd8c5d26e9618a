// quant.hip -- fused activation quantize + residue kernel (NVFP4 and MXFP4).
//
// One 256-thread workgroup per activation row.  Each thread owns 16-element
// slices j = tid + 256*c of the row and keeps them in registers for the whole
// kernel, so the row is read from HBM once:
//   1. row amax -> tensor scale s_g = amax / 2688 (NVFP4; ResServe Appendix B.2,
//      Eq. 8 with the maximum taken per row)
//   2. block scale: NVFP4 E4M3_RNE(blockmax / (6 s_g)), MXFP4 E8M0 from the
//      32-block maximum (Section 2, Figure 1)
//   3. element codes E2M1_RNE(v / s~) (Eq. 10), packed two per byte
//   4. residue r = v - fl(s~ e) kept in the same registers (Section 4.4: the
//      residue is formed in registers, no second read of x)
//   5. steps 1-3 again on r with its own row amax; the row goes to record M+m.
// A 16-element NVFP4 block is owned by one thread; a 32-element MXFP4 block
// spans an adjacent lane pair, whose maxima meet through one lane swap.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "codec.h"
#include "kernels.h"
#include "layout.h"

namespace rsfp4 {

namespace {

constexpr int kQThreads = 256;

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Workgroup-wide maximum of non-negative values; every thread gets the result.
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();                       // red may still be read from a prior call
    if (lane == 0) red[wid] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kQThreads / 64; ++i) r = fmaxf(r, red[i]);
    return r;
}

template <typename T>
__device__ __forceinline__ void load16(const T* p, float* v);

template <>
__device__ __forceinline__ void load16<float>(const float* p, float* v) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 t = q[i];
        v[4 * i + 0] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
}

template <>
__device__ __forceinline__ void load16<__hip_bfloat16>(const __hip_bfloat16* p, float* v) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint4 t = q[i];
        uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {       // bf16 -> fp32 is exact: shift into the high half
            v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
            v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
}

// Quantize the NCH slices held in v[] (in place: v becomes the residue) into the
// record at rec.  amax is the row maximum.
template <int FMT, int NCH>
__device__ __forceinline__ void quantize_slices(float (&v)[NCH][16], int nslices, int64_t K,
                                                float amax, uint8_t* rec) {
    const int tid = threadIdx.x;
    uint8_t* codes = rec + kActHead;
    uint8_t* scales = codes + K / 2;
    const float s_g = (FMT == kNV) ? amax / 2688.0f : 0.0f;
    if (tid == 0) *reinterpret_cast<uint4*>(rec) = make_uint4(__float_as_uint(s_g), 0u, 0u, 0u);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = tid + kQThreads * c;          // slice index (16 elements)
        const bool valid = j < nslices;
        float bm = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) bm = fmaxf(bm, fabsf(v[c][e]));
        float st;                                    // effective element scale
        uint32_t sbyte;
        if (FMT == kNV) {
            const float t = bm / (6.0f * s_g);
            sbyte = e4m3_encode(t);
            st = e4m3_val(sbyte) * s_g;
        } else {
            // the 32-block spans slices 2i, 2i+1 = lanes tid, tid^1 (same wave)
            const float other = __shfl_xor(bm, 1, 64);
            sbyte = e8m0_for_amax(fmaxf(bm, other));
            st = e8m0_val(sbyte);
        }
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float x = v[c][e];
            uint32_t mag = 0u;
            if (st != 0.0f) mag = e2m1_mag(fabsf(x / st));
            const uint32_t code = (__float_as_uint(x) >> 28 & 8u) | mag;
            packed[e >> 3] |= code << (4 * (e & 7));
            const float d = st * e2m1_val(code);
            v[c][e] = x - d;                          // residue, exact (Sterbenz)
        }
        if (valid) {
            *reinterpret_cast<uint2*>(codes + 8 * (int64_t)j) = make_uint2(packed[0], packed[1]);
            if (FMT == kNV) {
                scales[j] = (uint8_t)sbyte;
            } else if ((j & 1) == 0) {
                scales[j >> 1] = (uint8_t)sbyte;
            }
        }
    }
}

template <int FMT, int NCH, typename TIn>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(const TIn* __restrict__ x, int M,
                                                              int64_t K, int with_res,
                                                              uint8_t* __restrict__ act,
                                                              int64_t row_bytes) {
    __shared__ float red[kQThreads / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const int nslices = (int)(K / 16);
    const TIn* xr = x + (int64_t)m * K;

    float v[NCH][16];
    float tmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int j = tid + kQThreads * c;
        if (j < nslices) {
            load16<TIn>(xr + 16 * (int64_t)j, v[c]);
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) v[c][e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, fabsf(v[c][e]));
    }
    const float amax = block_max(tmax, red);
    quantize_slices<FMT, NCH>(v, nslices, K, amax, act + (int64_t)m * row_bytes);
    if (!with_res) return;

    // v now holds the residue (zero in invalid slices): second row statistic.
    float rmax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) rmax = fmaxf(rmax, fabsf(v[c][e]));
    const float ramax = block_max(rmax, red);
    quantize_slices<FMT, NCH>(v, nslices, K, ramax, act + (int64_t)(M + m) * row_bytes);
}

template <int FMT, int NCH, typename TIn>
hipError_t launch_quant_t(const void* x, int M, int64_t K, int with_res, void* act, hipStream_t s) {
    const int64_t rb = act_row_bytes(FMT, K);
    hipLaunchKernelGGL((quant_act_kernel<FMT, NCH, TIn>), dim3(M), dim3(kQThreads), 0, s,
                       static_cast<const TIn*>(x), M, K, with_res, static_cast<uint8_t*>(act), rb);
    return hipGetLastError();
}

template <int FMT, typename TIn>
hipError_t launch_quant_f(const void* x, int M, int64_t K, int with_res, void* act, hipStream_t s) {
    const int64_t nsl = K / 16;
    if (nsl <= 1 * kQThreads) return launch_quant_t<FMT, 1, TIn>(x, M, K, with_res, act, s);
    if (nsl <= 2 * kQThreads) return launch_quant_t<FMT, 2, TIn>(x, M, K, with_res, act, s);
    if (nsl <= 4 * kQThreads) return launch_quant_t<FMT, 4, TIn>(x, M, K, with_res, act, s);
    return launch_quant_t<FMT, 8, TIn>(x, M, K, with_res, act, s);
}

}  // namespace

hipError_t launch_quantize_act(int fmt, int xt_bf16, const void* x, int M, int64_t K, int with_res,
                               void* act, hipStream_t s) {
    if (fmt == kNV) {
        return xt_bf16 ? launch_quant_f<kNV, __hip_bfloat16>(x, M, K, with_res, act, s)
                       : launch_quant_f<kNV, float>(x, M, K, with_res, act, s);
    }
    return xt_bf16 ? launch_quant_f<kMX, __hip_bfloat16>(x, M, K, with_res, act, s)
                   : launch_quant_f<kMX, float>(x, M, K, with_res, act, s);
}

}  // namespace rsfp4
