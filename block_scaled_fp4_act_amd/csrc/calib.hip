// calib.hip -- calibration for selective compensation (K-Ext).
//
// ResServe, Appendix B.1 (Eq. 7): each channel is scored by its mean absolute
// activation over calibration data, and every group of 8 channels keeps the k
// best (k = 8 rho).  Both steps run once, offline; their result is the K/8
// mask bytes that the extended weight prepack and the extended quantizer take.
//
//   channel_abs_sum_kernel: one thread per channel walks the rows in order and
//     adds |x| in binary64, so the sum is the same however the grid is laid
//     out (a fixed row count orders channels as the mean does).  Adjacent
//     threads read adjacent channels of a row: each row step is one coalesced
//     read, eight of them in flight before the adds consume them.
//   kext_select_kernel: one thread per group ranks its 8 scores; channel j is
//     kept when fewer than k channels beat it (a higher score, or an equal score
//     at a lower index).
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "kernels.h"

namespace rsfp4 {

namespace {

template <typename T>
__device__ __forceinline__ double absd(const T* p, int64_t i);
template <>
__device__ __forceinline__ double absd<float>(const float* p, int64_t i) { return fabs((double)p[i]); }
template <>
__device__ __forceinline__ double absd<__hip_bfloat16>(const __hip_bfloat16* p, int64_t i) {
    const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
    return fabs((double)__uint_as_float((uint32_t)b << 16));
}

template <typename T>
__global__ __launch_bounds__(256) void channel_abs_sum_kernel(const T* __restrict__ x, int64_t T_rows,
                                                              int64_t K, double* __restrict__ sum,
                                                              int accumulate) {
    const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (i >= K) return;
    double s = accumulate ? sum[i] : 0.0;
    int64_t t = 0;
    for (; t + 8 <= T_rows; t += 8) {
        double a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = absd<T>(x, (t + u) * K + i);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += a[u];     // in row order
    }
    for (; t < T_rows; ++t) s += absd<T>(x, t * K + i);
    sum[i] = s;
}

__global__ __launch_bounds__(256) void kext_select_kernel(const double* __restrict__ score, int64_t G,
                                                          int k, uint8_t* __restrict__ masks) {
    const int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (g >= G) return;
    double s[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] = score[8 * g + j];
    uint32_t mask = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int beaten = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) beaten += (s[i] > s[j]) || (i < j && s[i] == s[j]);
        mask |= (beaten < k ? 1u : 0u) << j;
    }
    masks[g] = (uint8_t)mask;
}

}  // namespace

hipError_t launch_channel_abs_sum(int xt_bf16, const void* x, int64_t T, int64_t K, double* sum,
                                  int accumulate, hipStream_t s) {
    const unsigned blocks = (unsigned)((K + 255) / 256);
    if (xt_bf16)
        hipLaunchKernelGGL(channel_abs_sum_kernel<__hip_bfloat16>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const __hip_bfloat16*>(x), T, K, sum, accumulate);
    else
        hipLaunchKernelGGL(channel_abs_sum_kernel<float>, dim3(blocks), dim3(256), 0, s,
                           static_cast<const float*>(x), T, K, sum, accumulate);
    return hipGetLastError();
}

hipError_t launch_kext_select(const double* score, int64_t K, int k, uint8_t* masks, hipStream_t s) {
    const int64_t G = K / 8;
    const unsigned blocks = (unsigned)((G + 255) / 256);
    hipLaunchKernelGGL(kext_select_kernel, dim3(blocks), dim3(256), 0, s, score, G, k, masks);
    return hipGetLastError();
}

}  // namespace rsfp4
