// api.cpp -- the C ABI: host-side validation, size queries and dispatch.
// Nothing here computes on the host; every step of the path runs in the
// kernels of quant.hip, prepack.hip, calib.hip, gemm.hip and gemm_tile.hip.
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
constexpr int64_t kMaxNarrowK = 16384; // K of one narrow-M launch (16 waves x 8 steps)
constexpr int64_t kMaxLinearK = 32768;
constexpr int64_t kMaxQuantK = 32768;
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
    if (K > kMaxQuantK) return fail(RSFP4_ERR_SHAPE, "quantize needs K <= 32768 (K = %lld)", (long long)K);
    if (!aligned(x, 16) || !aligned(act, 16)) return fail(RSFP4_ERR_ALIGN, "x and act must be 16-byte aligned");
    const size_t need = (size_t)act_row_bytes(fmt, K) * (size_t)(with_res ? 2 * M : M);
    if (bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", bytes, need);
    int cus = 0;
    st = num_cus(&cus);
    if (st != RSFP4_OK) return st;
    return hip_status(launch_quantize_act(fmt, xt == RSFP4_BF16, x, (int)M, K, with_res ? 1 : 0, act, cus,
                                          (hipStream_t)stream),
                      "quantize launch");
}

// Workspace of the tiled products over rewritten activations: the counter
// area, then the tiled operand; 0 when that would exceed kMaxTileWs (the
// records path then runs without it).  An NVFP4 product with few tiles splits
// K into ks slices (nv_tile_split), whose partial sums follow the tiled
// operand at the next 256-byte boundary (tile_split_ws_bytes; 0 past
// kMaxTileWs: the product then runs unsplit).
constexpr int64_t kMaxTileWs = (int64_t)1 << 30;
int64_t tile_ws_bytes(int fmt, int64_t B, int64_t K) {
    const int64_t t = act_tile_bytes(fmt, B, K);
    return t > kMaxTileWs ? 0 : kSplitCounterBytes + t;
}
int64_t tile_part_offset(int fmt, int64_t B, int64_t K) {
    return kSplitCounterBytes + (act_tile_bytes(fmt, B, K) + 255) / 256 * 256;
}
int tile_split(int fmt, int64_t B, int64_t N, int64_t K, int cus) {
    return fmt == RSFP4_NVFP4 ? nv_tile_split(B, N, K, cus) : 1;
}
int64_t tile_split_ws_bytes(int fmt, bool comp, int64_t B, int64_t N, int64_t K, int ks) {
    if (ks <= 1) return tile_ws_bytes(fmt, B, K);
    const int64_t t = tile_part_offset(fmt, B, K) + nv_split_bytes(B, N, ks, comp);
    return t > kMaxTileWs ? 0 : t;
}

// Whether the linear takes the tiled kernel: above 32 operand rows B, except
// compensated NVFP4 with 33..64 rows, K <= 4096 and N <= 4096, which runs the
// narrow kernel with four row tiles in one launch, reading each weight step
// once (measured at M = 17 and 32, K = N = 4096: 12.9 and 15.1 us against
// 16.1 and 17.2 us tiled; but at K = 14336, N = 4096 the tiled product, split
// in K, takes 24.2 and 25.6 us against 50.7 and 61.8, and at K = 4096,
// N = 14336 19.9 and 21.2 us against 25.4 and 26.1); and bf16 output with K
// above one narrow launch, which cannot take the narrow kernel's second,
// accumulating launch (the tiled kernel makes one pass over K).
bool tiled_shape(int fmt, bool comp, int64_t B, int64_t N, int64_t K, bool out_bf16) {
    const bool narrow4 = fmt == RSFP4_NVFP4 && comp && B > kNarrowRows && B <= 2 * kNarrowRows && K <= 4096 &&
                         N <= 4096;
    return (B > kNarrowRows && !narrow4) || (out_bf16 && K > kMaxNarrowK);
}

// The narrow linear's plan for one launch over `steps` (split across
// workgroups where the shape gains from it: compensated NVFP4, see
// plan_gemm_small), its workspace bytes, and whether the caller's workspace
// allows the split (else the unsplit plan, the same result up to the
// summation order of the K slices).
GemmPlan narrow_plan(int fmt, bool comp, int64_t M, int64_t N, int64_t steps, int cus, bool single_pass,
                     size_t ws_bytes, int64_t* need) {
    const bool split_ok = fmt == RSFP4_NVFP4 && comp && single_pass;
    GemmPlan pl = plan_gemm_small(M, N, steps, comp, cus, split_ok);
    *need = split_ws_bytes(pl, comp, N);
    if (pl.ks > 1 && (size_t)*need > ws_bytes) pl = plan_gemm_small(M, N, steps, comp, cus, false);
    return pl;
}

rsfp4_status linear(int fmt, bool comp, const void* act, size_t act_bytes, const void* w_packed,
                    size_t w_bytes, int64_t M, int64_t N, int64_t K, void* y, bool out_bf16, void* ws,
                    size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!act || !w_packed || !y) return fail(RSFP4_ERR_NULL, "act, w_packed and y must be non-NULL");
    if (M < 1 || M > 65535) return fail(RSFP4_ERR_SHAPE, "M = %lld outside [1, 65535]", (long long)M);
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    if (K > kMaxLinearK) return fail(RSFP4_ERR_UNSUPPORTED, "the linear supports K <= %lld (K = %lld)",
                                     (long long)kMaxLinearK, (long long)K);
    const int64_t B = comp ? 2 * M : M;
    if (!aligned(act, 16) || !aligned(w_packed, 256) || !aligned(y, out_bf16 ? 2 : 4))
        return fail(RSFP4_ERR_ALIGN, "act must be 16-, w_packed 256- and y element aligned");
    if (ws == nullptr) ws_bytes = 0;
    if (ws_bytes > 0 && !aligned(ws, 256)) return fail(RSFP4_ERR_ALIGN, "ws must be 256-byte aligned");
    const int64_t rb = act_row_bytes(fmt, K);
    const size_t need_a = (size_t)rb * (size_t)B;
    if (act_bytes < need_a) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", act_bytes, need_a);
    const size_t need_w = (size_t)packed_weight_bytes(fmt, N, K);
    if (w_bytes < need_w) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, needs %zu", w_bytes, need_w);
    // The tiled kernel addresses the activation operand with 32-bit offsets
    // below its out-of-range marker 2^31.
    if (tiled_shape(fmt, comp, B, N, K, out_bf16)) {
        if ((int64_t)rb * B >= ((int64_t)1 << 31))
            return fail(RSFP4_ERR_UNSUPPORTED, "activation operand of %lld bytes: the linear needs < 2^31",
                        (long long)((int64_t)rb * B));
        if (std::getenv("RSFP4_LOG"))
            std::fprintf(stderr, "[rsfp4] linear fmt=%d comp=%d M=%lld N=%lld K=%lld tiled\n", fmt, (int)comp,
                         (long long)M, (long long)N, (long long)K);
        // With a workspace that holds the activation operand rewritten in tiles
        // (after the counter area, which stays zero; MXFP4: the packed-weight
        // layout, both operands then streamed into LDS; NVFP4: exact f16 MFMA
        // fragments, streamed into LDS) the activations arrive as contiguous
        // 1 KB requests; same bits as the records path
        // (and, with room for them, the K slices' partial sums of a split)
        const int64_t tws = tile_ws_bytes(fmt, B, K);
        if (tws > 0 && (int64_t)ws_bytes >= tws) {
            int cus = 0;
            st = num_cus(&cus);
            if (st != RSFP4_OK) return st;
            int ks = tile_split(fmt, B, N, K, cus);
            if (ks > 1) {
                const int64_t sws = tile_split_ws_bytes(fmt, comp, B, N, K, ks);
                if (sws == 0 || (int64_t)ws_bytes < sws) ks = 1;
            }
            uint8_t* wsb = static_cast<uint8_t*>(ws);
            void* at = wsb + kSplitCounterBytes;
            st = hip_status(launch_act_tile(fmt, comp, act, rb, (int)M, K, at, (hipStream_t)stream), "linear launch");
            if (st != RSFP4_OK) return st;
            if (fmt == RSFP4_NVFP4)
                return hip_status(
                    launch_gemm_tile_dma_nv(comp, at, act, rb, w_packed, (int)M, N, K, y, out_bf16, ks,
                                            reinterpret_cast<int*>(wsb),
                                            reinterpret_cast<float*>(wsb + tile_part_offset(fmt, B, K)),
                                            (hipStream_t)stream),
                    "linear launch");
            return hip_status(launch_gemm_tile_dma(comp, at, w_packed, (int)M, N, K, y, out_bf16, cus,
                                                   (hipStream_t)stream),
                              "linear launch");
        }
        return hip_status(launch_gemm_tile(fmt, comp, act, rb, w_packed, (int)M, N, K, y, out_bf16,
                                           (hipStream_t)stream),
                          "linear launch");
    }
    int cus = 0;
    st = num_cus(&cus);
    if (st != RSFP4_OK) return st;
    // one launch covers up to kMaxNarrowK; a longer K takes two launches over
    // consecutive step ranges (the first a multiple of 8 steps), the second
    // adding its part to y.  Compensated NVFP4 with two row tiles (B > 16)
    // runs launches of at most 32 steps (2 per wave), where the activation
    // fragments fit in registers as f16 (dequantized once, not at every use):
    // the extra launches and read-modify-writes of y cost less than the
    // dequantization they save.
    const int S = (int)num_steps(K);
    int chunk = S;
    if (K > kMaxNarrowK) {
        chunk = 8 * ((S + 15) / 16);
    } else if (fmt == RSFP4_NVFP4 && comp && B > 16 && !out_bf16 && S > 32) {
        // two row tiles with a workspace that holds the split's partial sums:
        // one pass with K split across workgroups in slices of 32 steps;
        // otherwise (and four row tiles, B > 32) launches of 32 steps
        int64_t need = 0;
        if (narrow_plan(fmt, comp, M, N, S, cus, true, ws_bytes, &need).ks <= 1) chunk = 32;
    }
    const int passes = (S + chunk - 1) / chunk;
    for (int pass = 0; pass < passes; ++pass) {
        const int s_lo = pass * chunk, s_hi = s_lo + chunk < S ? s_lo + chunk : S;
        int64_t need = 0;
        const GemmPlan pl = narrow_plan(fmt, comp, M, N, s_hi - s_lo, cus, passes == 1, ws_bytes, &need);
        if (std::getenv("RSFP4_LOG"))
            std::fprintf(stderr, "[rsfp4] linear fmt=%d comp=%d M=%lld N=%lld K=%lld steps=[%d,%d) rt=%d maxs=%d "
                         "kw=%d grid=%lld ngl=%d ks=%d\n", fmt, (int)comp, (long long)M, (long long)N, (long long)K,
                         s_lo, s_hi, pl.rt, pl.maxs, pl.kw, (long long)pl.grid, pl.ngl, pl.ks);
        st = hip_status(launch_gemm_small(fmt, pl, comp, act, rb, w_packed, (int)M, N, K, y, out_bf16, s_lo,
                                          s_hi, pass > 0, pl.ks > 1 ? ws : nullptr, (hipStream_t)stream),
                        "linear launch");
        if (st != RSFP4_OK) return st;
    }
    return RSFP4_OK;
}

// ---- grouped (mixture of experts) linear ----
rsfp4_status grouped_linear(int fmt, bool comp, const void* act, size_t act_bytes, int64_t M_total,
                            const void* w_packed, size_t w_bytes, int64_t E, const int32_t* offsets,
                            int64_t max_rows, int64_t N, int64_t K, float* y, void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!act || !w_packed || !offsets || !y) return fail(RSFP4_ERR_NULL, "act, w_packed, offsets and y must be non-NULL");
    if (M_total < 1 || M_total > 65535) return fail(RSFP4_ERR_SHAPE, "M_total = %lld outside [1, 65535]", (long long)M_total);
    if (E < 1 || E > 65535) return fail(RSFP4_ERR_SHAPE, "E = %lld outside [1, 65535]", (long long)E);
    if (max_rows < 1 || max_rows > M_total)
        return fail(RSFP4_ERR_SHAPE, "max_rows = %lld outside [1, M_total]", (long long)max_rows);
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    const int64_t B = comp ? 2 * max_rows : max_rows;
    if (B > kNarrowRows)
        return fail(RSFP4_ERR_UNSUPPORTED, "grouped linear: %lld operand rows per expert, at most %lld", (long long)B,
                    (long long)kNarrowRows);
    if (K > kMaxNarrowK)
        return fail(RSFP4_ERR_UNSUPPORTED, "grouped linear: K = %lld, at most %lld", (long long)K, (long long)kMaxNarrowK);
    if (!aligned(act, 16) || !aligned(w_packed, 256) || !aligned(offsets, 4) || !aligned(y, 4))
        return fail(RSFP4_ERR_ALIGN, "act 16-, w_packed 256-byte, offsets and y element aligned");
    const int64_t rb = act_row_bytes(fmt, K);
    const int64_t rows = comp ? 2 * M_total : M_total;
    if (rb * rows >= ((int64_t)1 << 31))
        return fail(RSFP4_ERR_UNSUPPORTED, "activation buffer of %lld bytes: needs < 2^31", (long long)(rb * rows));
    if (act_bytes < (size_t)(rb * rows))
        return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", act_bytes, (size_t)(rb * rows));
    const int64_t stride = packed_weight_bytes(fmt, N, K);
    if (w_bytes / (size_t)stride < (size_t)E)
        return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, %lld blobs need %zu", w_bytes, (long long)E,
                    (size_t)(stride * E));
    int cus = 0;
    st = num_cus(&cus);
    if (st != RSFP4_OK) return st;
    const int per_expert_cus = cus / E > 0 ? (int)(cus / E) : 1;
    const GemmPlan pl = plan_gemm_small(max_rows, N, num_steps(K), comp, per_expert_cus);
    return hip_status(launch_gemm_grouped(fmt, pl, comp, act, rb, (int)M_total, w_packed, stride, (int)E, offsets,
                                          (int)max_rows, N, K, y, (hipStream_t)stream),
                      "grouped linear launch");
}

// ---- quantize + linear from x in one call ----
bool from_x_one_launch(int fmt, bool comp, int64_t M) {
    return fmt == RSFP4_MXFP4 ? M <= 4 : (!comp && M <= 4);
}

rsfp4_status linear_from_x(int fmt, bool comp, const void* x, int xt, int64_t M, int64_t N, int64_t K,
                           const void* w_packed, size_t w_bytes, void* y, int yt, void* act, size_t act_bytes,
                           void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(fmt, K);
    if (st != RSFP4_OK) return st;
    if (!x || !w_packed || !y || !act) return fail(RSFP4_ERR_NULL, "x, w_packed, y and act must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown activation dtype %d", xt);
    if (yt != RSFP4_F32 && yt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown output dtype %d", yt);
    if (M < 1 || M > 65535) return fail(RSFP4_ERR_SHAPE, "M = %lld outside [1, 65535]", (long long)M);
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    if (K > kMaxQuantK) return fail(RSFP4_ERR_SHAPE, "quantize needs K <= 32768 (K = %lld)", (long long)K);
    const bool out_bf16 = yt == RSFP4_BF16;
    if (!aligned(x, 16) || !aligned(act, 16) || !aligned(w_packed, 256) || !aligned(y, out_bf16 ? 2 : 4))
        return fail(RSFP4_ERR_ALIGN, "x and act must be 16-, w_packed 256-byte and y element aligned");
    const size_t need_a = (size_t)act_row_bytes(fmt, K) * (size_t)(comp ? 2 * M : M);
    if (act_bytes < need_a) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", act_bytes, need_a);
    const size_t need_w = (size_t)packed_weight_bytes(fmt, N, K);
    if (w_bytes < need_w) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, needs %zu", w_bytes, need_w);
    // One launch where each workgroup's share of the quantization stays well
    // below the time its weights take to arrive (measured at K = 4096..8192,
    // same-box comparisons): MXFP4 (no divisions) with M <= 4, 10-13 % faster;
    // plain NVFP4 with M <= 4, 6-16 % faster.  Compensated NVFP4 quantizes
    // twice the rows with the division path: at M = 1..2 the two forms are
    // within run-to-run spread, from M = 4 the dedicated quantizer, spread
    // over M compute units, wins; it always takes two launches.
    if (xt == RSFP4_BF16 && from_x_one_launch(fmt, comp, M)) {
        int cus = 0;
        st = num_cus(&cus);
        if (st != RSFP4_OK) return st;
        const InqPlan q = plan_gemm_inq(fmt, M, N, K, comp, cus);
        if (q.ok) {
            if (std::getenv("RSFP4_LOG"))
                std::fprintf(stderr, "[rsfp4] linear_from_x fmt=%d comp=%d M=%lld N=%lld K=%lld one launch maxs=%d "
                             "kw=%d grid=%lld ngl=%d qrow=%d ncq=%d\n", fmt, (int)comp, (long long)M, (long long)N,
                             (long long)K, q.pl.maxs, q.pl.kw, (long long)q.pl.grid, q.pl.ngl, q.qrow, q.ncq);
            return hip_status(launch_gemm_inq(fmt, q, comp, x, w_packed, (int)M, N, K, y, out_bf16,
                                              (hipStream_t)stream),
                              "linear launch");
        }
    }
    st = quantize(fmt, x, xt, M, K, comp ? 1 : 0, act, act_bytes, stream);
    if (st != RSFP4_OK) return st;
    return linear(fmt, comp, act, act_bytes, w_packed, w_bytes, M, N, K, y, out_bf16, ws, ws_bytes, stream);
}

// ---- selective compensation (K-Ext) ----
// Extended width K + (K/8) k, or -1: k in {1, 2, 4, 8}, K a multiple of 32, and
// an extension of whole 32-element runs (so its blocks are whole in both formats).
int64_t kext_dim(int64_t K, int k) {
    if (k != 1 && k != 2 && k != 4 && k != 8) return -1;
    if (K < 32 || K % 32 != 0) return -1;
    const int64_t ext = (K / 8) * k;
    if (ext % 32 != 0) return -1;
    return K + ext;
}

rsfp4_status check_kext(int fmt, int64_t K, int k, int64_t* KE) {
    if (fmt != RSFP4_NVFP4 && fmt != RSFP4_MXFP4) return fail(RSFP4_ERR_FORMAT, "unknown format %d", fmt);
    if (k != 1 && k != 2 && k != 4 && k != 8)
        return fail(RSFP4_ERR_SHAPE, "k = %d: channels per 8-group must be 1, 2, 4 or 8", k);
    *KE = kext_dim(K, k);
    if (*KE < 0)
        return fail(RSFP4_ERR_SHAPE, "K = %lld with k = %d: K must be a multiple of 32 and K*k/8 of 32",
                    (long long)K, k);
    return RSFP4_OK;
}

rsfp4_status prepack_kext(int fmt, const void* W, int wt, int64_t N, int64_t K, const uint8_t* masks, int k,
                          void* w_packed, size_t bytes, void* stream) {
    g_err[0] = 0;
    int64_t KE = 0;
    rsfp4_status st = check_kext(fmt, K, k, &KE);
    if (st != RSFP4_OK) return st;
    if (!W || !w_packed || !masks) return fail(RSFP4_ERR_NULL, "W, masks and w_packed must be non-NULL");
    if (wt != RSFP4_F32 && wt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown weight dtype %d", wt);
    if (N < 1 || N > (int64_t)1 << 24) return fail(RSFP4_ERR_SHAPE, "N = %lld outside [1, 2^24]", (long long)N);
    if (KE > (int64_t)1 << 20) return fail(RSFP4_ERR_SHAPE, "K_eff = %lld above 2^20", (long long)KE);
    if (!aligned(w_packed, 256)) return fail(RSFP4_ERR_ALIGN, "w_packed must be 256-byte aligned");
    if (!aligned(W, 16)) return fail(RSFP4_ERR_ALIGN, "W must be 16-byte aligned");
    const size_t need = (size_t)packed_weight_bytes(fmt, N, KE);
    if (bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, needs %zu", bytes, need);
    return hip_status(launch_prepack_kext(fmt, wt == RSFP4_BF16, W, N, K, masks, k, w_packed, (hipStream_t)stream),
                      "prepack launch");
}

rsfp4_status quantize_kext(int fmt, const void* x, int xt, int64_t M, int64_t K, const uint8_t* masks, int k,
                           void* act, size_t bytes, void* stream) {
    g_err[0] = 0;
    int64_t KE = 0;
    rsfp4_status st = check_kext(fmt, K, k, &KE);
    if (st != RSFP4_OK) return st;
    if (!x || !act || !masks) return fail(RSFP4_ERR_NULL, "x, masks and act must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown activation dtype %d", xt);
    if (M < 1 || M > 65535) return fail(RSFP4_ERR_SHAPE, "M = %lld outside [1, 65535]", (long long)M);
    if (KE > kMaxQuantK) return fail(RSFP4_ERR_SHAPE, "K_eff = %lld above 32768", (long long)KE);
    if (!aligned(x, 16) || !aligned(act, 16)) return fail(RSFP4_ERR_ALIGN, "x and act must be 16-byte aligned");
    const size_t need = (size_t)act_row_bytes(fmt, KE) * (size_t)M;
    if (bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", bytes, need);
    return hip_status(launch_quantize_act_kext(fmt, xt == RSFP4_BF16, x, (int)M, K, masks, k, act,
                                               (hipStream_t)stream),
                      "quantize launch");
}

rsfp4_status quantize_alpha(const void* x, int xt, int64_t M, int64_t K, const float* alpha, int with_res,
                            void* act, size_t bytes, void* stream) {
    g_err[0] = 0;
    rsfp4_status st = check_common(RSFP4_NVFP4, K);
    if (st != RSFP4_OK) return st;
    if (!x || !act || !alpha) return fail(RSFP4_ERR_NULL, "x, alpha and act must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown activation dtype %d", xt);
    if (M < 1 || M > 65535) return fail(RSFP4_ERR_SHAPE, "M = %lld outside [1, 65535]", (long long)M);
    if (K > kMaxQuantK) return fail(RSFP4_ERR_SHAPE, "quantize needs K <= 32768 (K = %lld)", (long long)K);
    if (!aligned(x, 16) || !aligned(act, 16) || !aligned(alpha, 4))
        return fail(RSFP4_ERR_ALIGN, "x and act must be 16-byte and alpha 4-byte aligned");
    const size_t need = (size_t)act_row_bytes(RSFP4_NVFP4, K) * (size_t)(with_res ? 2 * M : M);
    if (bytes < need) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "act holds %zu bytes, needs %zu", bytes, need);
    return hip_status(launch_quantize_act_alpha(xt == RSFP4_BF16, x, (int)M, K, alpha, with_res ? 1 : 0, act,
                                                (hipStream_t)stream),
                      "quantize launch");
}

// ---- decode attention ----
bool attn_dims_ok(int64_t H_q, int64_t H_kv, int64_t D) {
    return (D == 128 || D == 256) && H_kv >= 1 && H_q >= H_kv && H_q % H_kv == 0 && H_q / H_kv <= 8 &&
           H_q <= 4096;
}

int64_t attn_ws_bytes(int64_t B, int64_t H_q, int64_t D, int splits) {
    return splits > 1 ? B * H_q * (int64_t)splits * (D + 2) * 4 : 0;
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
    g_err[0] = 0;
    if (check_common(fmt, K) != RSFP4_OK || M < 1 || M > 65535 || N < 1 || N > (int64_t)1 << 24 || K > kMaxLinearK)
        return 0;
    const int64_t B = compensated ? 2 * M : M;
    const int64_t S = num_steps(K);
    // wide operands on the tiled kernels: the rewritten activation operand
    // after the counter area
    int cus = 0;
    const bool have_cus = num_cus(&cus) == RSFP4_OK;
    if (tiled_shape(fmt, compensated != 0, B, N, K, false)) {
        // (without a device to count compute units on: the unsplit size)
        const int64_t sws =
            have_cus ? tile_split_ws_bytes(fmt, compensated != 0, B, N, K, tile_split(fmt, B, N, K, cus)) : 0;
        g_err[0] = 0;
        return (size_t)(sws > 0 ? sws : tile_ws_bytes(fmt, B, K));
    }
    // the split applies to one-pass plans of the narrow kernel with one or two
    // row tiles
    if (B > 32 || K > kMaxNarrowK || !have_cus) return 0;
    int64_t need = 0;
    (void)narrow_plan(fmt, compensated != 0, M, N, S, cus, true, (size_t)1 << 62, &need);
    return (size_t)need;
}

#define RSFP4_GROUPED(NAME, FMT, COMP)                                                                         \
    rsfp4_status NAME(const void* act, size_t act_bytes, int64_t M_total, const void* w_packed,              \
                      size_t w_packed_bytes, int64_t E, const int32_t* offsets, int64_t max_rows, int64_t N,  \
                      int64_t K, float* y, void* stream) {                                                    \
        return grouped_linear(FMT, COMP, act, act_bytes, M_total, w_packed, w_packed_bytes, E, offsets,      \
                              max_rows, N, K, y, stream);                                                     \
    }
RSFP4_GROUPED(rsfp4_nvfp4_grouped_linear, RSFP4_NVFP4, false)
RSFP4_GROUPED(rsfp4_nvfp4_grouped_linear_compensated, RSFP4_NVFP4, true)
RSFP4_GROUPED(rsfp4_mxfp4_grouped_linear, RSFP4_MXFP4, false)
RSFP4_GROUPED(rsfp4_mxfp4_grouped_linear_compensated, RSFP4_MXFP4, true)
#undef RSFP4_GROUPED

int rsfp4_from_x_launches(int fmt, int xt, int64_t M, int64_t N, int64_t K, int compensated) {
    g_err[0] = 0;
    if (check_common(fmt, K) != RSFP4_OK || (xt != RSFP4_F32 && xt != RSFP4_BF16) || M < 1 || M > 65535 || N < 1 ||
        N > (int64_t)1 << 24 || K > kMaxQuantK)
        return 0;
    if (xt != RSFP4_BF16 || !from_x_one_launch(fmt, compensated != 0, M)) return 2;
    int cus = 0;
    if (num_cus(&cus) != RSFP4_OK) return 0;
    return plan_gemm_inq(fmt, M, N, K, compensated != 0, cus).ok ? 1 : 2;
}

rsfp4_status rsfp4_nvfp4_linear_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K, const void* w_packed,
                 size_t w_packed_bytes, void* y, int yt, void* act, size_t act_bytes, void* ws,
                 size_t ws_bytes, void* stream) {
    return linear_from_x(RSFP4_NVFP4, false, x, xt, M, N, K, w_packed, w_packed_bytes, y, yt, act, act_bytes, ws, ws_bytes,
                         stream);
}
rsfp4_status rsfp4_nvfp4_linear_compensated_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K, const void* w_packed,
                 size_t w_packed_bytes, void* y, int yt, void* act, size_t act_bytes, void* ws,
                 size_t ws_bytes, void* stream) {
    return linear_from_x(RSFP4_NVFP4, true, x, xt, M, N, K, w_packed, w_packed_bytes, y, yt, act, act_bytes, ws, ws_bytes,
                         stream);
}
rsfp4_status rsfp4_mxfp4_linear_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K, const void* w_packed,
                 size_t w_packed_bytes, void* y, int yt, void* act, size_t act_bytes, void* ws,
                 size_t ws_bytes, void* stream) {
    return linear_from_x(RSFP4_MXFP4, false, x, xt, M, N, K, w_packed, w_packed_bytes, y, yt, act, act_bytes, ws, ws_bytes,
                         stream);
}
rsfp4_status rsfp4_mxfp4_linear_compensated_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K, const void* w_packed,
                 size_t w_packed_bytes, void* y, int yt, void* act, size_t act_bytes, void* ws,
                 size_t ws_bytes, void* stream) {
    return linear_from_x(RSFP4_MXFP4, true, x, xt, M, N, K, w_packed, w_packed_bytes, y, yt, act, act_bytes, ws, ws_bytes,
                         stream);
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
    return linear(RSFP4_NVFP4, false, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, false, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_nvfp4_linear_compensated(const void* act, size_t act_bytes, const void* w_packed,
                                            size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, float* y,
                                            void* ws, size_t ws_bytes, void* stream) {
    return linear(RSFP4_NVFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, false, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
    g_err[0] = 0;
    if (!src || !sink) return fail(RSFP4_ERR_NULL, "src and sink must be non-NULL");
    if (!aligned(src, 16) || !aligned(sink, 4)) return fail(RSFP4_ERR_ALIGN, "src must be 16- and sink 4-byte aligned");
    if (bytes % 16 != 0) return fail(RSFP4_ERR_SHAPE, "stream read of %zu bytes: a multiple of 16 is required", bytes);
    int cus = 0;
    const rsfp4_status st = num_cus(&cus);
    if (st != RSFP4_OK) return st;
    if (bytes > (size_t)cus * ((size_t)1 << 30))
        return fail(RSFP4_ERR_UNSUPPORTED, "stream read of %zu bytes: at most 1 GiB per compute unit", bytes);
    return hip_status(launch_stream_read(src, (int64_t)bytes, static_cast<uint32_t*>(sink), cus, (hipStream_t)stream),
                      "stream read launch");
}

rsfp4_status rsfp4_nvfp4_linear_compensated_noalloc(const void* act, size_t act_bytes, const void* w_packed,
                                                    size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                                    float* y, void* stream) {
    size_t need = rsfp4_workspace_bytes(RSFP4_NVFP4, M, N, K, 1);
    if (need > (size_t)scratch_bytes()) {
        // a wide operand's workspace holds its rewritten activations and a
        // split's partial sums, both optional (without the split: the same
        // result up to the summation order of the K slices; without the
        // rewrite: the records path, the same bits): run with what fits
        if (M >= 1 && tiled_shape(RSFP4_NVFP4, true, 2 * M, N, K, false))
            need = (size_t)scratch_bytes();
        else
            return fail(RSFP4_ERR_UNSUPPORTED, "this shape's split needs %zu bytes of workspace; the library's "
                        "scratch holds %lld (use rsfp4_nvfp4_linear_compensated with a workspace)", need,
                        (long long)scratch_bytes());
    }
    void* ws = nullptr;
    if (need > 0) {
        const rsfp4_status st = hip_status(scratch_ptr((hipStream_t)stream, &ws), "library scratch");
        if (st != RSFP4_OK) return st;
    }
    return linear(RSFP4_NVFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, false, ws, need, stream);
}
rsfp4_status rsfp4_mxfp4_linear(const void* act, size_t act_bytes, const void* w_packed, size_t w_packed_bytes,
                                int64_t M, int64_t N, int64_t K, float* y, void* ws, size_t ws_bytes,
                                void* stream) {
    return linear(RSFP4_MXFP4, false, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, false, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_linear_compensated(const void* act, size_t act_bytes, const void* w_packed,
                                            size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, float* y,
                                            void* ws, size_t ws_bytes, void* stream) {
    return linear(RSFP4_MXFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, false, ws, ws_bytes, stream);
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

rsfp4_status rsfp4_validate_packed(const void* w_packed, size_t w_packed_bytes, int* fmt, int64_t* N, int64_t* K,
                                   void* stream) {
    g_err[0] = 0;
    if (!w_packed) return fail(RSFP4_ERR_NULL, "w_packed must be non-NULL");
    if (!aligned(w_packed, 256)) return fail(RSFP4_ERR_ALIGN, "w_packed must be 256-byte aligned");
    if (w_packed_bytes < (size_t)kWHeader)
        return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, the header alone is %lld", w_packed_bytes,
                    (long long)kWHeader);
    WHeader h;
    hipError_t e = hipMemcpyAsync(&h, w_packed, sizeof h, hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "header copy");
    if (h.magic != kMagic) return fail(RSFP4_ERR_FORMAT, "not a packed weight blob (magic 0x%08x)", h.magic);
    if (h.abi_version != RSFP4_ABI_VERSION)
        return fail(RSFP4_ERR_FORMAT, "blob of ABI version %u, this library is %d", h.abi_version, RSFP4_ABI_VERSION);
    if (h.fmt != RSFP4_NVFP4 && h.fmt != RSFP4_MXFP4) return fail(RSFP4_ERR_FORMAT, "unknown format %u", h.fmt);
    if (check_common((int)h.fmt, h.K) != RSFP4_OK) return fail(RSFP4_ERR_FORMAT, "header K = %lld", (long long)h.K);
    if (h.N < 1 || h.N > (int64_t)1 << 24) return fail(RSFP4_ERR_FORMAT, "header N = %lld", (long long)h.N);
    const bool sg_ok = h.fmt == RSFP4_NVFP4 ? (h.s_g >= 0.0f && h.s_g < __builtin_inff()) : h.s_g == 0.0f;
    if (!sg_ok) return fail(RSFP4_ERR_FORMAT, "header tensor scale %g", (double)h.s_g);
    const size_t need = (size_t)packed_weight_bytes((int)h.fmt, h.N, h.K);
    if (w_packed_bytes < need)
        return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "w_packed holds %zu bytes, its header needs %zu", w_packed_bytes, need);
    if (fmt) *fmt = (int)h.fmt;
    if (N) *N = h.N;
    if (K) *K = h.K;
    return RSFP4_OK;
}

int64_t rsfp4_kext_dim(int64_t K, int k) { return kext_dim(K, k); }

rsfp4_status rsfp4_channel_abs_sum(const void* x, int xt, int64_t T, int64_t K, double* sum, int accumulate,
                                   void* stream) {
    g_err[0] = 0;
    if (!x || !sum) return fail(RSFP4_ERR_NULL, "x and sum must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown activation dtype %d", xt);
    if (T < 1 || K < 1 || K > (int64_t)1 << 24 || T > ((int64_t)1 << 40) / K)
        return fail(RSFP4_ERR_SHAPE, "T = %lld, K = %lld outside T >= 1, 1 <= K <= 2^24, T*K <= 2^40",
                    (long long)T, (long long)K);
    if (!aligned(sum, 8) || !aligned(x, xt == RSFP4_BF16 ? 2 : 4))
        return fail(RSFP4_ERR_ALIGN, "sum must be 8-byte and x element aligned");
    return hip_status(launch_channel_abs_sum(xt == RSFP4_BF16, x, T, K, sum, accumulate ? 1 : 0,
                                             (hipStream_t)stream),
                      "channel sum launch");
}

rsfp4_status rsfp4_kext_select(const double* score, int64_t K, int k, uint8_t* masks, void* stream) {
    g_err[0] = 0;
    if (!score || !masks) return fail(RSFP4_ERR_NULL, "score and masks must be non-NULL");
    if (k != 1 && k != 2 && k != 4 && k != 8)
        return fail(RSFP4_ERR_SHAPE, "k = %d: channels per 8-group must be 1, 2, 4 or 8", k);
    if (K < 8 || K % 8 != 0 || K > (int64_t)1 << 24)
        return fail(RSFP4_ERR_SHAPE, "K = %lld must be a multiple of 8 in [8, 2^24]", (long long)K);
    if (!aligned(score, 8)) return fail(RSFP4_ERR_ALIGN, "score must be 8-byte aligned");
    return hip_status(launch_kext_select(score, K, k, masks, (hipStream_t)stream), "select launch");
}

rsfp4_status rsfp4_nvfp4_prepack_weights_kext(const void* W, int wt, int64_t N, int64_t K, const uint8_t* masks,
                                              int k, void* w_packed, size_t w_packed_bytes, void* stream) {
    return prepack_kext(RSFP4_NVFP4, W, wt, N, K, masks, k, w_packed, w_packed_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_prepack_weights_kext(const void* W, int wt, int64_t N, int64_t K, const uint8_t* masks,
                                              int k, void* w_packed, size_t w_packed_bytes, void* stream) {
    return prepack_kext(RSFP4_MXFP4, W, wt, N, K, masks, k, w_packed, w_packed_bytes, stream);
}

rsfp4_status rsfp4_nvfp4_quantize_act_kext(const void* x, int xt, int64_t M, int64_t K, const uint8_t* masks,
                                           int k, void* act, size_t act_bytes, void* stream) {
    return quantize_kext(RSFP4_NVFP4, x, xt, M, K, masks, k, act, act_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_quantize_act_kext(const void* x, int xt, int64_t M, int64_t K, const uint8_t* masks,
                                           int k, void* act, size_t act_bytes, void* stream) {
    return quantize_kext(RSFP4_MXFP4, x, xt, M, K, masks, k, act, act_bytes, stream);
}

rsfp4_status rsfp4_nvfp4_tensor_alpha(const void* x, int xt, int64_t M, int64_t K, float* alpha, void* stream) {
    g_err[0] = 0;
    if (!x || !alpha) return fail(RSFP4_ERR_NULL, "x and alpha must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown activation dtype %d", xt);
    if (M < 1 || K < 1 || M > ((int64_t)1 << 40) / K)
        return fail(RSFP4_ERR_SHAPE, "M = %lld, K = %lld outside M, K >= 1, M*K <= 2^40", (long long)M, (long long)K);
    if (!aligned(alpha, 4) || !aligned(x, xt == RSFP4_BF16 ? 2 : 4))
        return fail(RSFP4_ERR_ALIGN, "alpha must be 4-byte and x element aligned");
    return hip_status(launch_tensor_alpha(xt == RSFP4_BF16, x, M * K, alpha, (hipStream_t)stream), "alpha launch");
}

rsfp4_status rsfp4_nvfp4_quantize_act_alpha(const void* x, int xt, int64_t M, int64_t K, const float* alpha,
                                            int with_residue, void* act, size_t act_bytes, void* stream) {
    return quantize_alpha(x, xt, M, K, alpha, with_residue, act, act_bytes, stream);
}

rsfp4_status rsfp4_nvfp4_linear_bf16(const void* act, size_t act_bytes, const void* w_packed, size_t w_packed_bytes,
                                     int64_t M, int64_t N, int64_t K, void* y, void* ws, size_t ws_bytes,
                                     void* stream) {
    return linear(RSFP4_NVFP4, false, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, true, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_nvfp4_linear_compensated_bf16(const void* act, size_t act_bytes, const void* w_packed,
                                                 size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, void* y,
                                                 void* ws, size_t ws_bytes, void* stream) {
    return linear(RSFP4_NVFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, true, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_linear_bf16(const void* act, size_t act_bytes, const void* w_packed, size_t w_packed_bytes,
                                     int64_t M, int64_t N, int64_t K, void* y, void* ws, size_t ws_bytes,
                                     void* stream) {
    return linear(RSFP4_MXFP4, false, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, true, ws, ws_bytes, stream);
}
rsfp4_status rsfp4_mxfp4_linear_compensated_bf16(const void* act, size_t act_bytes, const void* w_packed,
                                                 size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, void* y,
                                                 void* ws, size_t ws_bytes, void* stream) {
    return linear(RSFP4_MXFP4, true, act, act_bytes, w_packed, w_packed_bytes, M, N, K, y, true, ws, ws_bytes, stream);
}

size_t rsfp4_kv_page_bytes(int64_t H_kv, int64_t D) {
    if (H_kv < 1 || (D != 128 && D != 256)) return 0;
    return (size_t)kv_page_bytes(H_kv, D);
}

rsfp4_status rsfp4_kv_cache_write(const void* k, const void* v, int xt, int64_t T, int64_t H_kv, int64_t D,
                                  const int32_t* slots, float k_scale, float v_scale, void* cache, size_t cache_bytes,
                                  void* stream) {
    g_err[0] = 0;
    if (!k || !v || !slots || !cache) return fail(RSFP4_ERR_NULL, "k, v, slots and cache must be non-NULL");
    if (xt != RSFP4_F32 && xt != RSFP4_BF16) return fail(RSFP4_ERR_FORMAT, "unknown dtype %d", xt);
    if (H_kv < 1 || H_kv > 1024 || (D != 128 && D != 256))
        return fail(RSFP4_ERR_SHAPE, "H_kv = %lld, D = %lld: D must be 128 or 256", (long long)H_kv, (long long)D);
    if (T < 1 || T > ((int64_t)1 << 31) / (H_kv * 2 * (D / 16)))
        return fail(RSFP4_ERR_SHAPE, "T = %lld outside [1, 2^31 / (H_kv * D / 8)]", (long long)T);
    if (!(k_scale > 0.0f) || !(v_scale > 0.0f)) return fail(RSFP4_ERR_SHAPE, "k_scale and v_scale must be > 0");
    if (!aligned(cache, 256) || !aligned(k, 4) || !aligned(v, 4) || !aligned(slots, 4))
        return fail(RSFP4_ERR_ALIGN, "cache must be 256-byte, k, v and slots 4-byte aligned");
    const int64_t pb = kv_page_bytes(H_kv, D);
    const int64_t num_pages = (int64_t)(cache_bytes / (size_t)pb);
    if (num_pages < 1) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "cache holds %zu bytes, one page needs %lld", cache_bytes, (long long)pb);
    return hip_status(launch_kv_write(xt == RSFP4_BF16, k, v, slots, T, (int)H_kv, (int)D, k_scale, v_scale, cache,
                                      num_pages, (hipStream_t)stream),
                      "kv write launch");
}

int rsfp4_resattn_splits(int64_t B, int64_t H_kv, int64_t max_seq_len) {
    int cus = 0;
    if (num_cus(&cus) != RSFP4_OK || B < 1 || H_kv < 1 || max_seq_len < 1) return 1;
    return attn_auto_splits(B, H_kv, max_seq_len, cus);
}

size_t rsfp4_resattn_workspace_bytes(int64_t B, int64_t H_q, int64_t D, int splits) {
    if (B < 1 || H_q < 1 || (D != 128 && D != 256) || splits < 1) return 0;
    return (size_t)attn_ws_bytes(B, H_q, D, splits);
}

rsfp4_status rsfp4_resattn_decode(const void* q_act, size_t q_act_bytes, int compensated, const void* cache,
                                  size_t cache_bytes, const int32_t* block_table, int64_t max_pages,
                                  const int32_t* seq_lens, int64_t max_seq_len, int64_t B, int64_t H_q, int64_t H_kv,
                                  int64_t D, float k_scale, float v_scale, float sm_scale, int splits, void* out,
                                  int out_bf16, void* ws, size_t ws_bytes, void* stream) {
    g_err[0] = 0;
    if (!q_act || !cache || !block_table || !seq_lens || !out)
        return fail(RSFP4_ERR_NULL, "q_act, cache, block_table, seq_lens and out must be non-NULL");
    if (!attn_dims_ok(H_q, H_kv, D))
        return fail(RSFP4_ERR_SHAPE, "H_q = %lld, H_kv = %lld, D = %lld: D in {128, 256}, H_q a multiple of H_kv, "
                    "at most 8 query heads per KV head", (long long)H_q, (long long)H_kv, (long long)D);
    if (B < 1 || B > 65535 || max_pages < 1 || max_seq_len < 1 || max_seq_len > max_pages * 32 ||
        max_seq_len > ((int64_t)1 << 30))
        return fail(RSFP4_ERR_SHAPE, "B = %lld, max_pages = %lld, max_seq_len = %lld: need 1 <= B <= 65535 and "
                    "1 <= max_seq_len <= 32 * max_pages", (long long)B, (long long)max_pages, (long long)max_seq_len);
    int cus = 0;
    rsfp4_status st = num_cus(&cus);
    if (st != RSFP4_OK) return st;
    if (splits <= 0) splits = attn_auto_splits(B, H_kv, max_seq_len, cus);
    if (splits > 4096) return fail(RSFP4_ERR_SHAPE, "splits = %d above 4096", splits);
    if (!aligned(q_act, 16) || !aligned(cache, 256) || !aligned(out, out_bf16 ? 2 : 4) || !aligned(ws, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4))
        return fail(RSFP4_ERR_ALIGN, "q_act and ws 16-, cache 256-byte aligned; out and tables element aligned");
    const int64_t rb = act_row_bytes(RSFP4_NVFP4, D);
    const size_t need_q = (size_t)rb * (size_t)(B * H_q) * (compensated ? 2 : 1);
    if (q_act_bytes < need_q) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "q_act holds %zu bytes, needs %zu", q_act_bytes, need_q);
    const int64_t pb = kv_page_bytes(H_kv, D);
    const int64_t num_pages = (int64_t)(cache_bytes / (size_t)pb);
    if (num_pages < 1) return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "cache holds %zu bytes, one page needs %lld", cache_bytes, (long long)pb);
    const size_t need_ws = (size_t)attn_ws_bytes(B, H_q, D, splits);
    if (need_ws > 0 && (!ws || ws_bytes < need_ws))
        return fail(RSFP4_ERR_BUFFER_TOO_SMALL, "workspace holds %zu bytes, %d splits need %zu", ws_bytes, splits, need_ws);
    return hip_status(launch_resattn(q_act, rb, compensated ? 1 : 0, cache, num_pages, block_table, max_pages,
                                     seq_lens, (int)B, (int)H_q, (int)H_kv, (int)D, k_scale, v_scale, sm_scale,
                                     splits, max_seq_len, out, out_bf16 ? 1 : 0, static_cast<float*>(ws),
                                     (hipStream_t)stream),
                      "attention launch");
}

}  // extern "C"
