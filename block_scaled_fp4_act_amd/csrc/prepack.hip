// prepack.hip -- offline weight quantization into the tiled gfx950 layout.
//
// Weights are prepared once, before serving (ResServe, Section 5.4: weight
// preparation happens at export time; Figure 1c: weights are quantized offline).
// NVFP4 uses one tensor scale for the whole W (Appendix B.2, Eq. 8 with alpha
// taken over the tensor), MXFP4 one E8M0 scale per 32-block (Section 2).
//
// Three kernels: a one-thread header init, a max|W| reduction (NVFP4 only;
// atomicMax on the binary32 bits, which orders like the values for x >= 0, so
// the result does not depend on the order of arrival), and the pack kernel in
// which each thread quantizes one 16-element slice of one channel and writes its
// 8 code bytes and its scale byte straight to their tiled positions.  The
// selective-compensation variant packs [W | W_S] the same way, reading the
// extension slices through the channel masks.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "codec.h"
#include "kernels.h"
#include "layout.h"

namespace rsfp4 {

namespace {

__global__ void hdr_init_kernel(uint8_t* blob, int fmt, int64_t N, int64_t K) {
    WHeader* h = reinterpret_cast<WHeader*>(blob);
    h->magic = kMagic;
    h->abi_version = 1;
    h->fmt = (uint32_t)fmt;
    h->amax_bits = 0u;
    h->N = N;
    h->K = K;
    h->s_g = 0.0f;
    for (int i = 0; i < 7; ++i) h->pad[i] = 0u;
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<__hip_bfloat16>(const __hip_bfloat16* p, int64_t i) {
    const uint16_t b = reinterpret_cast<const uint16_t*>(p)[i];
    return __uint_as_float((uint32_t)b << 16);
}

template <typename T>
__global__ __launch_bounds__(256) void w_amax_kernel(const T* __restrict__ W, int64_t n,
                                                     uint8_t* blob) {
    float m = 0.0f;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        m = fmaxf(m, fabsf(ld<T>(W, i)));
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if ((threadIdx.x & 63) == 0) {
        WHeader* h = reinterpret_cast<WHeader*>(blob);
        atomicMax(&h->amax_bits, __float_as_uint(m));
    }
}

// Byte offsets inside the blob of the 8 code bytes of channel n, K-elements
// k0 .. k0+15 (k0 a multiple of 16), and of their block-scale byte.
__device__ __forceinline__ int64_t code_off(int fmt, int64_t K, int64_t n, int64_t k0) {
    const int64_t c = n / kGroupN, i = n % kGroupN;
    const int64_t s = k0 / kStepK, g = (k0 % kStepK) / 32, half = (k0 % 32) / 16;
    return kWHeader + c * group_bytes(fmt, K) + step_code_offset(fmt, s) + (g * 16 + i) * 16 + half * 8;
}
__device__ __forceinline__ int64_t scale_off(int fmt, int64_t K, int64_t n, int64_t k0) {
    const int64_t c = n / kGroupN, i = n % kGroupN;
    const int64_t s = k0 / kStepK, g = (k0 % kStepK) / 32, half = (k0 % 32) / 16;
    const int64_t lane = g * 16 + i;
    const int64_t base = kWHeader + c * group_bytes(fmt, K) + quad_scale_offset(fmt, s);
    if (fmt == kNV) return base + lane * 8 + (s % kQuadSteps) * 2 + half;
    return base + lane * 4 + (s % kQuadSteps);
}

// One thread per (channel n, 16-slice j) over the padded extent
// [16 * groups) x [128 * steps rounded up to whole quads / 16); MXFP4 pairs
// adjacent slices of one block through a lane swap (blockDim is a multiple of 64,
// slices are channel-major so slices 2t and 2t+1 of a channel sit in lanes 2u,
// 2u+1).  Slices of the padding steps of the last quad write zero codes and
// zero scales, so every byte a wave may load is defined.
// Selective compensation (ResServe Section 5.3, Eq. 6): the packed operand is
// [W | W_S], K = Kb + (Kb/8) k columns; column Kb + p is W's column of the
// (p % k)-th selected channel of group p / k (lowest channel first).  A mask
// byte with fewer than k bits falls back to the group's channel 7, in bounds.
__device__ __forceinline__ int64_t ext_column(const uint8_t* masks, int ks, int64_t p) {
    const int64_t g = p / ks;
    uint32_t rest = masks[g];
    for (int q = (int)(p % ks); q > 0; --q) rest &= rest - 1u;
    return 8 * g + (rest ? __builtin_ctz(rest) : 7);
}

template <int FMT, typename T>
__global__ __launch_bounds__(256) void prepack_kernel(const T* __restrict__ W, int64_t N, int64_t K,
                                                      uint8_t* __restrict__ blob, int64_t Kb,
                                                      const uint8_t* __restrict__ masks, int ks) {
    const WHeader* h = reinterpret_cast<const WHeader*>(blob);
    const int64_t S = num_steps(K);
    const int64_t S_pad = (S + kQuadSteps - 1) / kQuadSteps * kQuadSteps;
    const int64_t slices_per_row = S_pad * (kStepK / 16);
    const int64_t total = num_groups(N) * kGroupN * slices_per_row;
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    const bool live = t < total;
    const int64_t n = live ? t / slices_per_row : 0;
    const int64_t j = live ? t % slices_per_row : 0;
    const int64_t k0 = 16 * j;
    const bool real = live && n < N && k0 < K;   // K % 32 == 0: a slice is all in or all out

    // the slice's source columns: W's own for k0 < Kb, selected ones beyond
    // (Kb % 32 == 0: a 16-slice lies wholly on one side)
    float v[16];
    if (k0 < Kb || !real) {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = real ? ld<T>(W, n * Kb + k0 + e) : 0.0f;
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = ld<T>(W, n * Kb + ext_column(masks, ks, k0 + e - Kb));
    }
    float bm = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) bm = fmaxf(bm, fabsf(v[e]));

    float st;
    uint32_t sbyte;
    if (FMT == kNV) {
        const float s_g = __uint_as_float(h->amax_bits) / 2688.0f;
        if (t == 0) reinterpret_cast<WHeader*>(blob)->s_g = s_g;
        sbyte = e4m3_encode(bm / (6.0f * s_g));
        st = e4m3_val(sbyte) * s_g;
    } else {
        const float other = __shfl_xor(bm, 1, 64);
        sbyte = e8m0_for_amax(fmaxf(bm, other));
        st = e8m0_val(sbyte);
    }
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        uint32_t mag = 0u;
        if (st != 0.0f) mag = e2m1_mag(fabsf(v[e] / st));
        const uint32_t code = (__float_as_uint(v[e]) >> 28 & 8u) | mag;
        packed[e >> 3] |= code << (4 * (e & 7));
    }
    if (!real) { packed[0] = packed[1] = 0u; sbyte = 0u; }
    if (live) {
        *reinterpret_cast<uint2*>(blob + code_off(FMT, K, n, k0)) = make_uint2(packed[0], packed[1]);
        if (FMT == kNV || (j & 1) == 0) blob[scale_off(FMT, K, n, k0)] = (uint8_t)sbyte;
    }
}

// Inverse of the tiling, for tests: canonical codes [N, K/2] and scales [N, K/blk].
template <int FMT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ blob, int64_t N,
                                                     int64_t K, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, float* s_g) {
    const int64_t spr = K / 16;
    const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (t == 0 && s_g) *s_g = reinterpret_cast<const WHeader*>(blob)->s_g;
    if (t >= N * spr) return;
    const int64_t n = t / spr, j = t % spr, k0 = 16 * j;
    const uint2 c = *reinterpret_cast<const uint2*>(blob + code_off(FMT, K, n, k0));
    *reinterpret_cast<uint2*>(codes + n * (K / 2) + 8 * j) = c;
    if (FMT == kNV) {
        scales[n * (K / 16) + j] = blob[scale_off(FMT, K, n, k0)];
    } else if ((j & 1) == 0) {
        scales[n * (K / 32) + j / 2] = blob[scale_off(FMT, K, n, k0)];
    }
}

// K: columns of the packed operand; Kb: columns of W (K = Kb unless masks).
template <int FMT, typename T>
hipError_t prepack_t(const void* W, int64_t N, int64_t K, int64_t Kb, const uint8_t* masks, int ks,
                     void* blob, hipStream_t s) {
    uint8_t* b = static_cast<uint8_t*>(blob);
    hipLaunchKernelGGL(hdr_init_kernel, dim3(1), dim3(1), 0, s, b, FMT, N, K);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (FMT == kNV) {
        const int64_t n = N * Kb;   // the selected columns repeat W's: same maximum
        int64_t blocks = (n + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL((w_amax_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const T*>(W), n, b);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t S_pad = (num_steps(K) + kQuadSteps - 1) / kQuadSteps * kQuadSteps;
    const int64_t total = num_groups(N) * kGroupN * S_pad * (kStepK / 16);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL((prepack_kernel<FMT, T>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const T*>(W), N, K, b, Kb, masks, ks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prepack(int fmt, int wt_bf16, const void* W, int64_t N, int64_t K, void* blob,
                          hipStream_t s) {
    if (fmt == kNV)
        return wt_bf16 ? prepack_t<kNV, __hip_bfloat16>(W, N, K, K, nullptr, 0, blob, s)
                       : prepack_t<kNV, float>(W, N, K, K, nullptr, 0, blob, s);
    return wt_bf16 ? prepack_t<kMX, __hip_bfloat16>(W, N, K, K, nullptr, 0, blob, s)
                   : prepack_t<kMX, float>(W, N, K, K, nullptr, 0, blob, s);
}

hipError_t launch_prepack_kext(int fmt, int wt_bf16, const void* W, int64_t N, int64_t Kb,
                               const uint8_t* masks, int k, void* blob, hipStream_t s) {
    const int64_t K = Kb + (Kb / 8) * k;
    if (fmt == kNV)
        return wt_bf16 ? prepack_t<kNV, __hip_bfloat16>(W, N, K, Kb, masks, k, blob, s)
                       : prepack_t<kNV, float>(W, N, K, Kb, masks, k, blob, s);
    return wt_bf16 ? prepack_t<kMX, __hip_bfloat16>(W, N, K, Kb, masks, k, blob, s)
                   : prepack_t<kMX, float>(W, N, K, Kb, masks, k, blob, s);
}

hipError_t launch_unpack(int fmt, const void* blob, int64_t N, int64_t K, uint8_t* codes,
                         uint8_t* scales, float* s_g, hipStream_t s) {
    const int64_t total = N * (K / 16);
    const int64_t blocks = (total + 255) / 256;
    const uint8_t* b = static_cast<const uint8_t*>(blob);
    if (fmt == kNV)
        hipLaunchKernelGGL(unpack_kernel<kNV>, dim3((unsigned)blocks), dim3(256), 0, s, b, N, K,
                           codes, scales, s_g);
    else
        hipLaunchKernelGGL(unpack_kernel<kMX>, dim3((unsigned)blocks), dim3(256), 0, s, b, N, K,
                           codes, scales, s_g);
    return hipGetLastError();
}

}  // namespace rsfp4
