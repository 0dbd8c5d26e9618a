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
constexpr int kRedBytesMax = 128 * 1024;   // LDS for partial sums per workgroup
constexpr int kLdsPerCu = 160 * 1024;      // gfx950

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit dwords, range checked

// NVFP4 block-scale pair -> two f16 holding S_b * 2^-8 each.  E4M3 (bias 7) and
// f16 (bias 15) line up field by field: the E4M3 exponent and mantissa bits
// moved to f16's exponent and top mantissa bits give the same value times 2^-8,
// subnormals included.  The 2^8 comes back through the conversion's power-of-
// two scale below, so e * S_b is formed exactly.
__device__ __forceinline__ half2v scale_pair_h(uint32_t two_bytes) {
    const uint32_t bits = ((two_bytes & 0x7Fu) << 7) | ((two_bytes & 0x7F00u) << 15);
    return __builtin_bit_cast(half2v, bits);
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

__device__ __forceinline__ uint32_t get(const uint4& v, int u) {
    return u == 0 ? v.x : (u == 1 ? v.y : (u == 2 ? v.z : v.w));
}

__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

struct GemmArgs {
    const uint8_t* act;
    int64_t row_bytes;
    const uint8_t* blob;
    int M;
    int64_t N;
    int64_t K;
    float* y;
    int ngl;          // groups whose partial sums are held in LDS between reductions
};

// APRE: the activation fragments are dequantized to f16 once, before the
// weight stream starts (NVFP4 only; 16 VGPRs per step and row tile), so the
// streaming loop only dequantizes weights.  Without it they stay as codes and
// are dequantized at each use.
// PD: weight prefetch depth.  The loads of group j + PD are issued before group
// j is computed, through a ring of PD + 1 register buffers (the loop is
// unrolled by PD + 1 so every buffer index is static); PD = 0 loads each group
// just before its use.
template <int FMT, int MAXS, int RT, bool COMP, int PD, bool APRE>
__global__ __launch_bounds__(1024) void gemm_small_kernel(GemmArgs p) {
    extern __shared__ float red[];           // [ngl][KW][RT][4][64] partial sums
    constexpr bool kPre = APRE && FMT == kNV;
    constexpr int kAC = kPre ? 1 : MAXS;     // code registers kept per row tile
    constexpr int kAH = kPre ? MAXS : 1;     // f16 fragments kept per row tile
    constexpr int NB = PD + 1;               // weight buffers in the ring

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
    constexpr uint32_t SB = (uint32_t)step_bytes(FMT);
    const uint32_t scale_base = (uint32_t)(kActHead + p.K / 2);
    const int64_t grid = gridDim.x;
    const int64_t c0 = blockIdx.x;

    float s_gw = 1.0f;
    if (FMT == kNV) s_gw = reinterpret_cast<const WHeader*>(p.blob)->s_g;

    uint4 wb[NB][MAXS];
    uint32_t wsc[NB][MAXS];

    // One buffer resource per group (32-bit lane offsets, no 4 GB limit
    // overall).  Every load is issued unconditionally: a step past this wave's
    // range, or a group past the end (zero-sized resource), reads out of range
    // and the buffer unit returns zeros.  Without branches around the loads the
    // compiler's memory-counter waits stay exact, so prefetched groups are
    // really in flight while earlier ones are computed.
    auto load_w = [&](int64_t c, uint4 (&codes)[MAXS], uint32_t (&sc)[MAXS]) {
        const bool live = c < G;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.blob + kWHeader + (live ? c : 0) * GB), (short)0, live ? (int)GB : 0, kRsrcWord3);
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            const bool in = t < ns;
            const uint32_t st = (uint32_t)(s0 + t) * SB;
            codes[t] = ld128(r, in ? st + 16u * lane : (uint32_t)GB);
            if (FMT == kNV)
                sc[t] = __builtin_amdgcn_raw_buffer_load_b16(r, in ? st + (uint32_t)kStepCodes + 2u * lane : (uint32_t)GB, 0, 0);
            else
                sc[t] = __builtin_amdgcn_raw_buffer_load_b8(r, in ? st + (uint32_t)kStepCodes + lane : (uint32_t)GB, 0, 0);
        }
    };

    // ---- activation fragments: loaded once, kept in registers ----
    // Their loads go out first; the first groups' weight loads follow at once,
    // so both latencies overlap and the fragments can be dequantized while the
    // weights are still in flight.
    const int B = COMP ? 2 * p.M : p.M;
    const uint32_t act_bytes = (uint32_t)(B * p.row_bytes);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.act, (short)0, (int)act_bytes, kRsrcWord3);
    uint4 a_raw[RT][MAXS];
    uint32_t a_rsc[RT][MAXS];
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
            const bool in = t < ns && rvalid && k0 < p.K;   // else: out of range -> zeros
            const uint32_t rec = in ? (uint32_t)(arow * p.row_bytes) : act_bytes;
            a_raw[rt][t] = ld128(ra, in ? rec + (uint32_t)(kActHead + k0 / 2) : act_bytes);
            if (FMT == kNV)
                a_rsc[rt][t] = __builtin_amdgcn_raw_buffer_load_b16(ra, in ? rec + scale_base + (uint32_t)(k0 / 16) : act_bytes, 0, 0);
            else
                a_rsc[rt][t] = __builtin_amdgcn_raw_buffer_load_b8(ra, in ? rec + scale_base + (uint32_t)(k0 / 32) : act_bytes, 0, 0);
        }
    }

    if (PD == 0) {
        load_w(c0, wb[0], wsc[0]);
    } else {
#pragma unroll
        for (int q = 0; q < PD; ++q) load_w(c0 + q * grid, wb[q], wsc[q]);
    }


    uint4 a_codes[RT][kAC];
    uint32_t a_sc[RT][kAC];
    half8 a_h[RT][kAH][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (kPre) {
                const half2v h = scale_pair_h(a_rsc[rt][t]);
#pragma unroll
                for (int u = 0; u < 4; ++u) a_h[rt][t][u] = dequant8(get(a_raw[rt][t], u), u < 2 ? h[0] : h[1]);
            } else {
                a_codes[rt][t] = a_raw[rt][t];
                a_sc[rt][t] = a_rsc[rt][t];
            }
        }
    }

    // ---- one group: MFMAs over this wave's steps; partial sums to LDS slot ----
    auto compute = [&](int slot, const uint4 (&w_codes)[MAXS], const uint32_t (&w_sc)[MAXS]) {
        floatx4 acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (t < ns) {
                if (FMT == kNV) {
                    const half2v sw = scale_pair_h(w_sc[t]);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const half8 b = dequant8(get(w_codes[t], u), u < 2 ? sw[0] : sw[1]);
#pragma unroll
                        for (int rt = 0; rt < RT; ++rt) {
                            half8 a;
                            if (kPre) {
                                a = a_h[rt][t][u];
                            } else {
                                const half2v sa = scale_pair_h(a_sc[rt][t]);
                                a = dequant8(get(a_codes[rt][t], u), u < 2 ? sa[0] : sa[1]);
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
        float* dst = red + ((slot * KW + wave) * RT) * 256;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(rt * 4 + r) * 64 + lane] = acc[rt][r];
    };

    // ---- reduce the slots [0, nslots) of groups c_first, c_first + grid, ...:
    // sum the KW partials in a fixed order (deterministic), Fold, store ----
    auto flush = [&](int64_t c_first, int nslots) {
        __syncthreads();
        const int items = nslots * RT * 128;
        for (int idx = threadIdx.x; idx < items; idx += blockDim.x) {
            const int slot = idx / (RT * 128);
            const int rem = idx - slot * (RT * 128);
            const int rt = rem >> 7;
            const int pr = (rem >> 6) & 1;
            const int ln = rem & 63;
            const float* src = red + (slot * KW * RT + rt) * 256 + (2 * pr) * 64 + ln;
            float v0 = 0.0f, v1 = 0.0f;
            for (int w = 0; w < KW; ++w) {
                v0 += src[w * RT * 256];
                v1 += src[w * RT * 256 + 64];
            }
            const int og = ln >> 4, oi = ln & 15;
            const int ti0 = 16 * rt + 4 * og + 2 * pr;   // tile rows ti0, ti0 + 1
            const int64_t n = (c_first + slot * grid) * kGroupN + oi;
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
    };

    // groups of this workgroup: c0, c0 + grid, ...; the loop runs a whole number
    // of ring turns and skips the work (never the loads) past the end.  Partial
    // sums of up to ngl groups wait in LDS and are reduced together, so the
    // waves meet at a barrier once per ngl groups, not per group.
    const int64_t nj = c0 < G ? (G - c0 + grid - 1) / grid : 0;
    const int ngl = p.ngl;
    int slot = 0;
    if (PD == 0) {
        for (int64_t j = 0; j < nj; ++j) {
            if (j > 0) load_w(c0 + j * grid, wb[0], wsc[0]);
            compute(slot, wb[0], wsc[0]);
            if (++slot == ngl || j == nj - 1) {
                flush(c0 + (j - slot + 1) * grid, slot);
                slot = 0;
            }
        }
    } else {
        for (int64_t j0 = 0; j0 < nj; j0 += NB) {
#pragma unroll
            for (int q = 0; q < NB; ++q) {
                const int64_t j = j0 + q;
                load_w(c0 + (j + PD) * grid, wb[(q + PD) % NB], wsc[(q + PD) % NB]);
                if (j < nj) {
                    compute(slot, wb[q], wsc[q]);
                    if (++slot == ngl || j == nj - 1) {
                        flush(c0 + (j - slot + 1) * grid, slot);
                        slot = 0;
                    }
                }
            }
        }
    }
}

template <int FMT, int MAXS, int RT, bool COMP, int PD, bool APRE>
hipError_t launch_t(const GemmArgs& a, int KW, int64_t grid, hipStream_t s) {
    // allow the full LDS of a CU for the partial-sum slots (set once per kernel)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_small_kernel<FMT, MAXS, RT, COMP, PD, APRE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kRedBytesMax);
    if (attr != hipSuccess) return attr;
    const size_t lds = (size_t)a.ngl * KW * RT * 1024;
    hipLaunchKernelGGL((gemm_small_kernel<FMT, MAXS, RT, COMP, PD, APRE>), dim3((unsigned)grid),
                       dim3(64 * KW), lds, s, a);
    return hipGetLastError();
}

// Register budget (128 VGPRs at 16 waves per CU) decides the variant: each
// prefetch level costs one more set of weight registers (5 per step), the f16
// activation fragments 16 per step and row tile (NVFP4), the code fragments 5.
// The table below was chosen from the compiler's register counts so that no
// variant with one row tile spills; with two row tiles (B > 16) and 6-8 steps
// per wave a few registers spill.
constexpr int pd_for(int fmt, int rt, int maxs) {
    if (fmt == kNV && rt == 1) return maxs <= 2 ? 3 : (maxs <= 4 ? 2 : (maxs == 5 ? 1 : 0));
    if (fmt == kNV) return maxs == 1 ? 3 : (maxs == 2 ? 2 : (maxs <= 4 ? 1 : 0));
    if (rt == 1) return maxs <= 4 ? 3 : (maxs == 5 ? 2 : (maxs == 6 ? 1 : 0));
    return maxs <= 3 ? (maxs == 2 ? 2 : 3) : (maxs == 4 ? 1 : 0);
}
constexpr bool apre_for(int fmt, int rt, int maxs) { return fmt == kNV && rt == 1 && maxs <= 3; }

template <int FMT, int RT, bool COMP, int MAXS>
hipError_t launch_v(const GemmArgs& a, int KW, int64_t grid, hipStream_t s) {
    return launch_t<FMT, MAXS, RT, COMP, pd_for(FMT, RT, MAXS), apre_for(FMT, RT, MAXS)>(a, KW, grid, s);
}

template <int FMT, int RT, bool COMP>
hipError_t launch_maxs(const GemmArgs& a, int maxs, int KW, int64_t grid, hipStream_t s) {
    switch (maxs) {
        case 1: return launch_v<FMT, RT, COMP, 1>(a, KW, grid, s);
        case 2: return launch_v<FMT, RT, COMP, 2>(a, KW, grid, s);
        case 3: return launch_v<FMT, RT, COMP, 3>(a, KW, grid, s);
        case 4: return launch_v<FMT, RT, COMP, 4>(a, KW, grid, s);
        case 5: return launch_v<FMT, RT, COMP, 5>(a, KW, grid, s);
        case 6: return launch_v<FMT, RT, COMP, 6>(a, KW, grid, s);
        case 7: return launch_v<FMT, RT, COMP, 7>(a, KW, grid, s);
        default: return launch_v<FMT, RT, COMP, 8>(a, KW, grid, s);
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
    const int64_t per_wg = (G + pl.grid - 1) / pl.grid;         // groups per workgroup
    // LDS per workgroup: at most 128 KB, and small enough for per_cu of them
    const int64_t lds_cap = kRedBytesMax < kLdsPerCu / per_cu ? kRedBytesMax : kLdsPerCu / per_cu;
    const int64_t fit = lds_cap / ((int64_t)pl.kw * pl.rt * 1024);
    pl.ngl = (int)(per_wg < fit ? per_wg : fit);
    return pl;
}

hipError_t launch_gemm_small(int fmt, const GemmPlan& pl, bool comp, const void* act,
                             int64_t row_bytes, const void* blob, int M, int64_t N, int64_t K,
                             float* y, hipStream_t s) {
    GemmArgs a{static_cast<const uint8_t*>(act), row_bytes, static_cast<const uint8_t*>(blob), M,
               N, K, y, pl.ngl};
    if (fmt == kNV) return launch_fmt<kNV>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s);
    return launch_fmt<kMX>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s);
}

}  // namespace rsfp4
