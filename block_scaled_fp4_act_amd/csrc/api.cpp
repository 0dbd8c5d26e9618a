// api.cpp -- the C ABI: host-side validation, size queries and dispatch.
// Nothing here computes on the host; every step of the path runs in the
// kernels of quant.hip, prepack.hip and gemm.hip.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/rsfp4.h"
#include "kernels.h"
#include "layout.h"

using namespace rsfp4;

namespace {

thread_local char g_err[512] = "";

rsfp4_status fail(rsfp4_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

rsfp4_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return RSFP4_OK;
    return fail(RSFP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int kMaxDevices = 64;
constexpr int64_t kNarrowRows = 32;   // tile rows (base + residue) the narrow-M kernel handles
std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];

// Compute-unit count of the current device (cached per device).
rsfp4_status num_cus(int* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(RSFP4_ERR_UNSUPPORTED, "device %d", dev);
    std::call_once(g_cu_once[dev], [dev] {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
        g_cus[dev] = n;
    });
    if (g_cus[dev] <= 0) return fail(RSFP4_ERR_HIP, "could not query the compute-unit count of device %d", dev);
    *out = g_cus[dev];
    return RSFP4_OK;
}

rsfp4_status check_common(int fmt, int64_t K) {
    if (fmt != RSFP4_NVFP4 && fmt != RSFP4_MXFP4) return fail(RSFP4_ERR_FORMAT, "unknown format %d", fmt);
    if (K < 32 || K % 32 != 0) return fail(RSFP4_ERR_SHAPE, "K = %lld must be a positive multiple of 32", (long long)K);
    return RSFP4_OK;
}

rsfp4_status prepack(int fmt, const void* W, int wt, int64_t N, int64_t K, void* w_packed,
                     size_t bytes, void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!W || !w_packed) return fail(RSFP4_ERR_NULL, "W and w_packed must be non-NULL");
    if (wt != RSFP4_F32 && wt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown weight dtype %d", wt);
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    if (K > (int64_t)1 << 20) return fail(RSFP4_ERR_SHAPE, "K = %lld above 2^20", (long long)K);
    if (!aligned(w_packed, 256)) return fail(RSFP4_ERR_ALIGN, "w_packed must be 256-byte aligned");
    if (!aligned(W, 16)) return fail(RSFP4_ERR_ALIGN, "W must be 16-byte aligned");
    const size_t need = (size_t)packed_weight_bytes(fmt, N, K);
    if (bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, needs %zu", bytes, need);
    return hip_status(launch_prepack(fmt, wt == RSFP4_BF16, W, N, K, w_packed, (hipStream_t)stream),
                      "prepack launch");
}

rsfp4_status quantize(int fmt, const void* x, int xt, int64_t M, int64_t K, int with_res, void* act,
                      size_t bytes, void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!x || !act) return fail(RSFP4_ERR_NULL, "x and act must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown activation dtype %d", xt);
    if (M < 1 || M > 65535) return fail(RSFP4_ERR_SHAPE, "M = %lld outside [1, 65535]", (long long)M);
    if (K > 32768) return fail(RSFP4_ERR_SHAPE, "quantize needs K <= 32768 (K = %lld)", (long long)K);
    if (!aligned(x, 16) || !aligned(act, 16)) return fail(RSFP4_ERR_ALIGN, "x and act must be 16-byte aligned");
    const size_t need = (size_t)act_row_bytes(fmt, K) * (size_t)(with_res ? 2 * M : M);
    if (bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", bytes, need);
    return hip_status(launch_quantize_act(fmt, xt == RSFP4_BF16, x, (int)M, K, with_res ? 1 : 0, act,
                                          (hipStream_t)stream),
                      "quantize launch");
}

rsfp4_status linear(int fmt, bool comp, const void* act, size_t act_bytes, const void* w_packed,
                    size_t w_bytes, int64_t M, int64_t N, int64_t K, float* y, void* ws,
                    size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!act || !w_packed || !y) return fail(RSFP4_ERR_NULL, "act, w_packed and y must be non-NULL");
    if (M < 1 || M > 65535) return fail(RSFP4_ERR_SHAPE, "M = %lld outside [1, 65535]", (long long)M);
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    if (K > 16384) return fail(RSFP4_ERR_UNSUPPORTED, "the linear supports K <= 16384 (K = %lld)", (long long)K);
    const int64_t B = comp ? 2 * M : M;
    if (!aligned(act, 16) || !aligned(w_packed, 256) || !aligned(y, 4))
        return fail(RSFP4_ERR_ALIGN, "act must be 16-, w_packed 256- and y 4-byte aligned");
    const int64_t rb = act_row_bytes(fmt, K);
    const size_t need_a = (size_t)rb * (size_t)B;
    if (act_bytes < need_a) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", act_bytes, need_a);
    const size_t need_w = (size_t)packed_weight_bytes(fmt, N, K);
    if (w_bytes < need_w) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, needs %zu", w_bytes, need_w);
    if (B > kNarrowRows) {
        if (std::getenv("RSFP4_LOG"))
            std::fprintf(stderr, "[rsfp4] linear fmt=%d comp=%d M=%lld N=%lld K=%lld tiled\n", fmt, (int)comp,
                         (long long)M, (long long)N, (long long)K);
        return hip_status(launch_gemm_tile(fmt, comp, act, rb, w_packed, (int)M, N, K, y, (hipStream_t)stream),
                          "linear launch");
    }
    int cus = 0;
    st = num_cus(&cus);
    if (st != RSFP4_OK) return st;
    const GemmPlan pl = plan_gemm_small(M, N, K, comp, cus);
    if (std::getenv("RSFP4_LOG"))
        std::fprintf(stderr, "[rsfp4] linear fmt=%d comp=%d M=%lld N=%lld K=%lld rt=%d maxs=%d kw=%d grid=%lld ngl=%d\n",
                     fmt, (int)comp, (long long)M, (long long)N, (long long)K, pl.rt, pl.maxs, pl.kw,
                     (long long)pl.grid, pl.ngl);
    return hip_status(launch_gemm_small(fmt, pl, comp, act, rb,
                                        w_packed, (int)M, N, K, y, (hipStream_t)stream),
                      "linear launch");
}

}  // namespace

extern "C" {

int rsfp4_abi_version(void) { return RSFP4_ABI_VERSION; }

const char* rsfp4_status_string(int s) {
    switch (s) {
        case RSFP4_OK: return "ok";
        case RSFP4_ERR_NULL: return "null pointer";
        case RSFP4_ERR_SHAPE: return "bad shape";
        case RSFP4_ERR_ALIGN: return "misaligned buffer";
        case RSFP4_ERR_FORMAT: return "unknown format or dtype";
        case RSFP4_ERR_BUFFER_TOO_SMALL: return "buffer too small";
        case RSFP4_ERR_UNSUPPORTED: return "unsupported";
        case RSFP4_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* rsfp4_last_error(void) { return g_err; }

size_t rsfp4_act_row_bytes(int fmt, int64_t K) {
    if ((fmt != RSFP4_NVFP4 && fmt != RSFP4_MXFP4) || K < 32 || K % 32) return 0;
    return (size_t)act_row_bytes(fmt, K);
}

size_t rsfp4_packed_act_bytes(int fmt, int64_t M, int64_t K, int with_residue) {
    if (M < 1) return 0;
    return rsfp4_act_row_bytes(fmt, K) * (size_t)(with_residue ? 2 * M : M);
}

size_t rsfp4_packed_weight_bytes(int fmt, int64_t N, int64_t K) {
    if ((fmt != RSFP4_NVFP4 && fmt != RSFP4_MXFP4) || K < 32 || K % 32 || N < 1) return 0;
    return (size_t)packed_weight_bytes(fmt, N, K);
}

size_t rsfp4_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int compensated) {
    (void)fmt; (void)M; (void)N; (void)K; (void)compensated;
    return 0;
}

rsfp4_status rsfp4_nvfp4_prepack_weights(const void* W, int wt, int64_t N, int64_t K, void* w_packed,
                                         size_t w_packed_bytes, void* stream) {
    return prepack(RSFP4_NVFP4, W, wt, N, K, w_packed, w_packed_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_prepack_weights(const void* W, int wt, int64_t N, int64_t K, void* w_packed,
                                         size_t w_packed_bytes, void* stream) {
    return prepack(RSFP4_MXFP4, W, wt, N, K, w_packed, w_packed_bytes, stream);
}

rsfp4_status rsfp4_nvfp4_quantize_act_with_residue(const void* x, int xt, int64_t M, int64_t K,
                                                   int with_residue, void* act, size_t act_bytes,
                                                   void* stream) {
    return quantize(RSFP4_NVFP4, x, xt, M, K, with_residue, act, act_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_quantize_act_with_residue(const void* x, int xt, int64_t M, int64_t K,
                                                   int with_residue, void* act, size_t act_bytes,
                                                   void* stream) {
    return quantize(RSFP4_MXFP4, x, xt, M, K, with_residue, act, act_bytes, stream);
}

rsfp4_status rsfp4_nvfp4_linear(const void* act, size_t act_bytes, const void* w_packed, size_t w_packed_bytes,
                                int64_t M, int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                                void* stream) {
    return linear(RSFP4_NVFP4, false, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_nvfp4_linear_compensated(const void* act, size_t act_bytes, const void* w_packed,
                                            size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, float* y,
                                            void* ws, size_t ws_bytes, void* stream) {
    return linear(RSFP4_NVFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_linear(const void* act, size_t act_bytes, const void* w_packed, size_t w_packed_bytes,
                                int64_t M, int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                                void* stream) {
    return linear(RSFP4_MXFP4, false, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_linear_compensated(const void* act, size_t act_bytes, const void* w_packed,
                                            size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, float* y,
                                            void* ws, size_t ws_bytes, void* stream) {
    return linear(RSFP4_MXFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, ws, ws_bytes, stream);
}

rsfp4_status rsfp4_unpack_weights_canonical(const void* w_packed, size_t w_packed_bytes, int fmt, int64_t N,
                                            int64_t K, uint8_t* codes, uint8_t* scales, float* s_g,
                                            void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!w_packed || !codes || !scales) return fail(RSFP4_ERR_NULL, "w_packed, codes and scales must be non-NULL");
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    if (!aligned(w_packed, 256) || !aligned(codes, 8)) return fail(RSFP4_ERR_ALIGN, "w_packed 256-, codes 8-byte aligned");
    const size_t need = (size_t)packed_weight_bytes(fmt, N, K);
    if (w_packed_bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, needs %zu", w_packed_bytes, need);
    return hip_status(launch_unpack(fmt, w_packed, N, K, codes, scales, s_g, (hipStream_t)stream), "unpack launch");
}

}  // extern "C"
