// gemm.hip -- narrow-M block-scaled FP4 linear on the gfx950 matrix cores,
// plain (B = M activation rows) and residue-compensated (B = 2M rows).
//
// What is computed (ResServe, arXiv 2611.08713, Section 4.2 Eq. 1 and Section
// 4.3 Eq. 2): Z = [X^; R^] W^T with the Fold Y_j = Z_j + Z_{M+j}.  The swap of
// Section 5.1 (Eq. 4) is about which MMA output dimension the tokens occupy; on
// gfx950 the 16x16 MFMA tile is square, so the choice here is the one that puts
// a token's base and residue row in the same lane: activation rows are the MFMA
// A operand (output rows), ordered base/residue interleaved (tile row 2m = q(x)
// row m, 2m+1 = q(r) row m), and each lane of the 16x16 accumulator holds tile
// rows 4g..4g+3 of one channel, i.e. two complete pairs -- the Fold is a
// thread-local fp32 add before the only store (the idea of the row-pair packing
// of Figure 5, realised with MFMA lane ownership instead of TMEM loads).
//
// Work decomposition (one design for all M <= 16, i.e. B <= 32):
//   * a workgroup owns groups of 16 output channels (grid-stride over groups)
//     and has KW waves that split K: wave w owns a contiguous run of <= MAXS
//     128-element steps;
//   * a wave loads its activation fragments for its steps ONCE (they stay in
//     VGPRs across all groups), then streams the packed weights: per step one
//     16-byte load per lane = 1 KB per wave, fully coalesced, plus the step's
//     scales; the next group's weights are prefetched while the current group
//     computes, so every weight byte is read from HBM once;
//   * NVFP4: each 8-element run is dequantized in registers to f16 with its
//     E4M3 block scale (e * S_b has <= 6 significant bits and lies in
//     [2^-10, 2688], so f16 holds it exactly) and fed to
//     v_mfma_f32_16x16x32_f16; the fp32 tensor scales s_gx, s_gr, s_gw are
//     applied in the Fold epilogue;
//   * MXFP4: codes and E8M0 scales go straight into the native block-scaled
//     v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4, one scale per lane = per
//     32-element block), no dequantization at all;
//   * the KW partial accumulators of a group meet in LDS and are summed in a
//     fixed order (deterministic), then folded and stored as fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.h"
#include "kernels.h"
#include "layout.h"

namespace rsfp4 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));

constexpr int kMaxWaves = 16;

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times an
// E4M3 block scale -> eight exact f16.  The gfx950 scaled conversion applies only
// the exponent of its fp32 scale operand (a power-of-two scale, as MX formats
// need), so it converts with unit scale and the full E4M3 scale is applied with
// a packed f16 multiply; every product e * S_b is representable in f16, so the
// multiply is exact.
__device__ __forceinline__ half8 dequant8(uint32_t w, _Float16 scale) {
    half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    const half2v s2 = {scale, scale};
    p0 *= s2; p1 *= s2; p2 *= s2; p3 *= s2;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

__device__ __forceinline__ _Float16 e4m3_h(uint32_t b) { return (_Float16)e4m3_val(b); }

__device__ __forceinline__ uint32_t get(const uint4& v, int u) {
    return u == 0 ? v.x : (u == 1 ? v.y : (u == 2 ? v.z : v.w));
}

struct GemmArgs {
    const uint8_t* act;
    int64_t row_bytes;
    const uint8_t* blob;
    int M;
    int64_t N;
    int64_t K;
    float* y;
};

// APRE: the activation fragments are dequantized to f16 once, before the
// weight stream starts (NVFP4 only; costs 16 VGPRs per step and row tile), so
// the streaming loop only dequantizes weights.  Without it they stay as codes
// and are dequantized at each use.
template <int FMT, int MAXS, int RT, bool COMP, bool PREF, bool APRE>
__global__ __launch_bounds__(1024) void gemm_small_kernel(GemmArgs p) {
    __shared__ float red[kMaxWaves * RT * 4 * 64];
    constexpr bool kPre = APRE && FMT == kNV;
    constexpr int kAC = kPre ? 1 : MAXS;     // code registers kept per row tile
    constexpr int kAH = kPre ? MAXS : 1;     // f16 fragments kept per row tile

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int KW = blockDim.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int64_t S = num_steps(p.K);
    const int s0 = (int)((wave * S) / KW);
    const int s1 = (int)(((wave + 1) * S) / KW);
    const int ns = s1 - s0;                       // <= MAXS by the host's choice
    const int64_t G = num_groups(p.N);
    const int64_t GB = group_bytes(FMT, p.K);
    constexpr int64_t SB = step_bytes(FMT);
    const int64_t scale_base = kActHead + p.K / 2;

    // ---- activation fragments: loaded once, kept in registers ----
    uint4 a_codes[RT][kAC];
    uint32_t a_sc[RT][kAC];
    half8 a_h[RT][kAH][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int ti = 16 * rt + i;               // tile row of this lane's A operand
        int arow;
        bool rvalid;
        if (COMP) {
            const int m = ti >> 1;
            rvalid = m < p.M;
            arow = (ti & 1) ? p.M + m : m;
        } else {
            rvalid = ti < p.M;
            arow = ti;
        }
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            const int64_t k0 = kStepK * (s0 + t) + 32 * g;
            uint4 cd = make_uint4(0u, 0u, 0u, 0u);
            uint32_t sc = 0u;
            if (t < ns && rvalid && k0 < p.K) {
                const uint8_t* rec = p.act + (int64_t)arow * p.row_bytes;
                cd = *reinterpret_cast<const uint4*>(rec + kActHead + k0 / 2);
                if (FMT == kNV)
                    sc = *reinterpret_cast<const uint16_t*>(rec + scale_base + k0 / 16);
                else
                    sc = rec[scale_base + k0 / 32];
            }
            if (kPre) {
                const _Float16 h0 = e4m3_h(sc & 0xFFu), h1 = e4m3_h(sc >> 8);
#pragma unroll
                for (int u = 0; u < 4; ++u) a_h[rt][t][u] = dequant8(get(cd, u), u < 2 ? h0 : h1);
            } else {
                a_codes[rt][t] = cd;
                a_sc[rt][t] = sc;
            }
        }
    }

    float s_gw = 1.0f;
    if (FMT == kNV) s_gw = reinterpret_cast<const WHeader*>(p.blob)->s_g;

    uint4 w_codes[MAXS], n_codes[MAXS];
    uint32_t w_sc[MAXS], n_sc[MAXS];

    auto load_w = [&](int64_t c, uint4 (&codes)[MAXS], uint32_t (&sc)[MAXS]) {
        const uint8_t* gb = p.blob + kWHeader + c * GB;
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (t < ns) {
                const uint8_t* st = gb + (int64_t)(s0 + t) * SB;
                codes[t] = *reinterpret_cast<const uint4*>(st + 16 * lane);
                if (FMT == kNV)
                    sc[t] = *reinterpret_cast<const uint16_t*>(st + kStepCodes + 2 * lane);
                else
                    sc[t] = st[kStepCodes + lane];
            } else {
                codes[t] = make_uint4(0u, 0u, 0u, 0u);
                sc[t] = 0u;
            }
        }
    };

    int64_t c = blockIdx.x;
    if (c < G) load_w(c, w_codes, w_sc);

    for (; c < G; c += gridDim.x) {
        const int64_t cn = c + gridDim.x;
        if (PREF && cn < G) load_w(cn, n_codes, n_sc);

        floatx4 acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (t < ns) {
                if (FMT == kNV) {
                    const _Float16 sw0 = e4m3_h(w_sc[t] & 0xFFu);
                    const _Float16 sw1 = e4m3_h(w_sc[t] >> 8);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const half8 b = dequant8(get(w_codes[t], u), u < 2 ? sw0 : sw1);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            half8 a;
                            if (kPre) {
                                a = a_h[rt][t][u];
                            } else {
                                const uint32_t sb = u < 2 ? (a_sc[rt][t] & 0xFFu) : (a_sc[rt][t] >> 8);
                                a = dequant8(get(a_codes[rt][t], u), e4m3_h(sb));
                            }
                            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[rt], 0, 0, 0);
                        }
                    }
                } else {
                    const uint4 wc = w_codes[t];
                    const intx8 b = {(int)wc.x, (int)wc.y, (int)wc.z, (int)wc.w, 0, 0, 0, 0};
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        const uint4 ac = a_codes[rt][t];
                        const intx8 a = {(int)ac.x, (int)ac.y, (int)ac.z, (int)ac.w, 0, 0, 0, 0};
                        acc[rt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            a, b, acc[rt], 4, 4, 0, (int)a_sc[rt][t], 0, (int)w_sc[t]);
                    }
                }
            }
        }

        // ---- cross-wave reduction in LDS, fixed order, then Fold + store ----
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[((wave * RT + rt) * 4 + r) * 64 + lane] = acc[rt][r];
        __syncthreads();
        for (int idx = threadIdx.x; idx < RT * 128; idx += blockDim.x) {
            const int rt = idx >> 7;
            const int pr = (idx >> 6) & 1;
            const int ln = idx & 63;
            float v0 = 0.0f, v1 = 0.0f;
            for (int w = 0; w < KW; ++w) {
                v0 += red[((w * RT + rt) * 4 + 2 * pr) * 64 + ln];
                v1 += red[((w * RT + rt) * 4 + 2 * pr + 1) * 64 + ln];
            }
            const int og = ln >> 4, oi = ln & 15;
            const int ti0 = 16 * rt + 4 * og + 2 * pr;   // tile rows ti0, ti0 + 1
            const int64_t n = c * kGroupN + oi;
            if (n < p.N) {
                if (COMP) {
                    const int m = ti0 >> 1;
                    if (m < p.M) {
                        float out;
                        if (FMT == kNV) {
                            const float sx = *reinterpret_cast<const float*>(p.act + (int64_t)m * p.row_bytes);
                            const float sr = *reinterpret_cast<const float*>(p.act + (int64_t)(p.M + m) * p.row_bytes);
                            out = s_gw * (sx * v0 + sr * v1);
                        } else {
                            out = v0 + v1;
                        }
                        p.y[(int64_t)m * p.N + n] = out;
                    }
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int m = ti0 + h;
                        if (m < p.M) {
                            const float v = h ? v1 : v0;
                            float out = v;
                            if (FMT == kNV)
                                out = s_gw * (*reinterpret_cast<const float*>(p.act + (int64_t)m * p.row_bytes) * v);
                            p.y[(int64_t)m * p.N + n] = out;
                        }
                    }
                }
            }
        }
        __syncthreads();

        if (PREF) {
#pragma unroll
            for (int t = 0; t < MAXS; ++t) { w_codes[t] = n_codes[t]; w_sc[t] = n_sc[t]; }
        } else if (cn < G) {
            load_w(cn, w_codes, w_sc);
        }
    }
}

template <int FMT, int MAXS, int RT, bool COMP, bool PREF, bool APRE>
hipError_t launch_t(const GemmArgs& a, int KW, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_small_kernel<FMT, MAXS, RT, COMP, PREF, APRE>), dim3((unsigned)grid),
                       dim3(64 * KW), 0, s, a);
    return hipGetLastError();
}

// Register budget (128 VGPRs at 16 waves per CU) decides the variant: the
// next-group prefetch doubles the weight registers, the f16 activation
// fragments take 16 VGPRs per step and row tile.
template <int FMT, int RT, bool COMP>
hipError_t launch_maxs(const GemmArgs& a, int maxs, int KW, int64_t grid, hipStream_t s) {
    switch (maxs) {
        case 1: return launch_t<FMT, 1, RT, COMP, true, true>(a, KW, grid, s);
        case 2: return launch_t<FMT, 2, RT, COMP, true, RT == 1>(a, KW, grid, s);
        case 3: return launch_t<FMT, 3, RT, COMP, true, RT == 1>(a, KW, grid, s);
        case 4: return launch_t<FMT, 4, RT, COMP, true, false>(a, KW, grid, s);
        case 5: return launch_t<FMT, 5, RT, COMP, false, false>(a, KW, grid, s);
        case 6: return launch_t<FMT, 6, RT, COMP, false, false>(a, KW, grid, s);
        case 7: return launch_t<FMT, 7, RT, COMP, false, false>(a, KW, grid, s);
        default: return launch_t<FMT, 8, RT, COMP, false, false>(a, KW, grid, s);
    }
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, int rt, bool comp, int maxs, int KW, int64_t grid,
                      hipStream_t s) {
    if (rt == 1)
        return comp ? launch_maxs<FMT, 1, true>(a, maxs, KW, grid, s)
                    : launch_maxs<FMT, 1, false>(a, maxs, KW, grid, s);
    return comp ? launch_maxs<FMT, 2, true>(a, maxs, KW, grid, s)
                : launch_maxs<FMT, 2, false>(a, maxs, KW, grid, s);
}

}  // namespace

GemmPlan plan_gemm_small(int64_t M, int64_t N, int64_t K, bool comp, int num_cus) {
    GemmPlan pl;
    const int64_t S = num_steps(K);
    const int64_t B = comp ? 2 * M : M;
    pl.rt = B <= 16 ? 1 : 2;
    // as many waves along K as allowed (16), then the fewest steps per wave
    pl.maxs = (int)((S + kMaxWaves - 1) / kMaxWaves);
    pl.kw = (int)((S + pl.maxs - 1) / pl.maxs);
    const int per_cu = kMaxWaves / pl.kw > 0 ? kMaxWaves / pl.kw : 1;
    const int64_t G = num_groups(N);
    const int64_t cap = (int64_t)num_cus * per_cu;
    pl.grid = G < cap ? G : cap;
    return pl;
}

hipError_t launch_gemm_small(int fmt, const GemmPlan& pl, bool comp, const void* act,
                             int64_t row_bytes, const void* blob, int M, int64_t N, int64_t K,
                             float* y, hipStream_t s) {
    GemmArgs a{static_cast<const uint8_t*>(act), row_bytes, static_cast<const uint8_t*>(blob), M,
               N, K, y};
    if (fmt == kNV) return launch_fmt<kNV>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s);
    return launch_fmt<kMX>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s);
}

}  // namespace rsfp4
