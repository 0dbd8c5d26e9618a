// gemm_tile.hip -- block-scaled FP4 linear for wide activation operands
// (B > 32 rows: prefill-like M, or many decode rows), on the gfx950 matrix cores.
//
// Same operation as the narrow-M kernel (ResServe, arXiv 2611.08713, Section
// 4.2 Eq. 1 and Section 4.3 Eq. 2: Z = [X^; R^] W^T with the Fold
// Y_j = Z_j + Z_{M+j}), but the tile is dense, so the work is split as a
// classic 2-D tiling instead of across K: a workgroup of 4 waves owns 128
// activation tile rows x 128 output channels; each wave owns a 64 x 64
// quarter = 4 x 4 MFMA tiles of 16 x 16 and walks all of K, streaming its
// activation fragments (4 row tiles) and weight fragments (4 channel groups,
// straight from the packed layout: one 1 KB load per group and step is exactly
// one MFMA operand) with a one-step-ahead register prefetch.
//   * MXFP4: native v_mfma_scale_f32_16x16x128_f8f6f4, FP4 x FP4 with the E8M0
//     block scales of both operands (the "really dense" case of the scaled
//     FP4 MFMA);
//   * NVFP4: exact f16 dequantization (e * S_b, see the narrow-M kernel) and
//     v_mfma_f32_16x16x32_f16; the tensor scales are applied in the Fold.
// Tile rows interleave base and residue rows (2m = q(x) row m, 2m+1 = q(r) row
// m), so every accumulator lane holds complete pairs and the Fold is a
// thread-local add before the only store.
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;     // raw buffer, 32-bit dwords, range checked
constexpr int kTileRows = 128;             // activation tile rows per workgroup
constexpr int kTileCh = 128;               // output channels per workgroup

__device__ __forceinline__ _Float16 scale_h(uint32_t byte) {
    // E4M3 byte -> S_b * 2^-8 as f16 (fields line up; see the narrow-M kernel)
    return __builtin_bit_cast(_Float16, (unsigned short)((byte & 0x7Fu) << 7));
}

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

struct TileArgs {
    const uint8_t* act;
    int64_t row_bytes;
    const uint8_t* blob;
    int M;
    int64_t N;
    int64_t K;
    float* y;
};

// One K-step (128 elements) of operands for a wave: 4 activation row tiles and
// 4 weight channel groups, codes (16 bytes per lane) and scale bytes.
struct Step {
    uint4 a[4];
    uint32_t as[4];
    uint4 b[4];
    uint32_t bs[4];
};

template <int FMT, bool COMP>
__global__ __launch_bounds__(256) void gemm_tile_kernel(TileArgs p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wr = wave >> 1, wc = wave & 1;
    const int g = lane >> 4, i = lane & 15;
    const int64_t S = num_steps(p.K);
    const int64_t G = num_groups(p.N);
    const int64_t GB = group_bytes(FMT, p.K);
    const uint32_t scale_base = (uint32_t)(kActHead + p.K / 2);
    const int B = COMP ? 2 * p.M : p.M;
    const uint32_t act_bytes = (uint32_t)(B * p.row_bytes);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.act, (short)0, (int)act_bytes, kRsrcWord3);

    // this lane's activation rows (one per row tile) and weight groups
    uint32_t arec[4];
    bool avalid[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int R = kTileRows * blockIdx.y + 64 * wr + 16 * rt + i;
        int arow;
        bool ok;
        if (COMP) {
            const int m = R >> 1;
            ok = m < p.M;
            arow = (R & 1) ? p.M + m : m;
        } else {
            ok = R < p.M;
            arow = R;
        }
        avalid[rt] = ok;
        arec[rt] = ok ? (uint32_t)(arow * p.row_bytes) : act_bytes;
    }
    __amdgpu_buffer_rsrc_t rw[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int64_t c = (int64_t)(kTileCh / 16) * blockIdx.x + 4 * wc + ct;
        const bool live = c < G;
        rw[ct] = __builtin_amdgcn_make_buffer_rsrc((void*)(p.blob + kWHeader + (live ? c : 0) * GB),
                                                  (short)0, live ? (int)GB : 0, kRsrcWord3);
    }

    // every load is unconditional (out of range -> zeros) so the compiler's
    // memory-counter waits stay exact across the prefetch
    auto load = [&](int64_t s, Step& st) {
        const int64_t k0 = kStepK * s + 32 * g;
        const bool kin = s < S && k0 < p.K;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const bool in = kin && avalid[rt];
            st.a[rt] = ld128(ra, in ? arec[rt] + (uint32_t)(kActHead + k0 / 2) : act_bytes);
            if (FMT == kNV)
                st.as[rt] = __builtin_amdgcn_raw_buffer_load_b16(ra, in ? arec[rt] + scale_base + (uint32_t)(k0 / 16) : act_bytes, 0, 0);
            else
                st.as[rt] = __builtin_amdgcn_raw_buffer_load_b8(ra, in ? arec[rt] + scale_base + (uint32_t)(k0 / 32) : act_bytes, 0, 0);
        }
        const uint32_t coff = s < S ? (uint32_t)step_code_offset(FMT, s) + 16u * lane : (uint32_t)GB;
        const uint32_t soff = s < S ? (uint32_t)(quad_scale_offset(FMT, s) + lane * 4 * scale_bytes_per_step_lane(FMT) +
                                                 (s % 4) * scale_bytes_per_step_lane(FMT))
                                    : (uint32_t)GB;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            st.b[ct] = ld128(rw[ct], coff);
            if (FMT == kNV)
                st.bs[ct] = __builtin_amdgcn_raw_buffer_load_b16(rw[ct], soff, 0, 0);
            else
                st.bs[ct] = __builtin_amdgcn_raw_buffer_load_b8(rw[ct], soff, 0, 0);
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[rt][ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](const Step& st) {
        if (FMT == kNV) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                half8 bh[4], ah[4];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    bh[ct] = dequant8(get(st.b[ct], u), scale_h((st.bs[ct] >> (u < 2 ? 0 : 8)) & 0xFFu));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    ah[rt] = dequant8(get(st.a[rt], u), scale_h((st.as[rt] >> (u < 2 ? 0 : 8)) & 0xFFu));
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bh[ct], acc[rt][ct], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const intx8 a = {(int)st.a[rt].x, (int)st.a[rt].y, (int)st.a[rt].z, (int)st.a[rt].w, 0, 0, 0, 0};
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const intx8 b = {(int)st.b[ct].x, (int)st.b[ct].y, (int)st.b[ct].z, (int)st.b[ct].w, 0, 0, 0, 0};
                    acc[rt][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        a, b, acc[rt][ct], 4, 4, 0, (int)st.as[rt], 0, (int)st.bs[ct]);
                }
            }
        }
    };

    // K loop with a two-step register ring (unrolled by two: static indices)
    Step ring[2];
    load(0, ring[0]);
    for (int64_t s = 0; s < S; s += 2) {
        load(s + 1, ring[1]);
        compute(ring[0]);
        load(s + 2, ring[0]);
        if (s + 1 < S) compute(ring[1]);
    }

    // Fold + store: lane holds tile rows 16rt + 4g + r of channel 16ct + i
    float s_gw = 1.0f;
    if (FMT == kNV) s_gw = reinterpret_cast<const WHeader*>(p.blob)->s_g;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int64_t n = (int64_t)kTileCh * blockIdx.x + 64 * wc + 16 * ct + i;
            if (n >= p.N) continue;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const int R0 = kTileRows * blockIdx.y + 64 * wr + 16 * rt + 4 * g + 2 * pr;
                const float v0 = acc[rt][ct][2 * pr], v1 = acc[rt][ct][2 * pr + 1];
                if (COMP) {
                    const int m = R0 >> 1;
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
                        const int m = R0 + h;
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
    }
}

template <int FMT, bool COMP>
hipError_t launch_tile_t(const TileArgs& a, hipStream_t s) {
    const int B = COMP ? 2 * a.M : a.M;
    const dim3 grid((unsigned)((a.N + kTileCh - 1) / kTileCh), (unsigned)((B + kTileRows - 1) / kTileRows));
    hipLaunchKernelGGL((gemm_tile_kernel<FMT, COMP>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_tile(int fmt, bool comp, const void* act, int64_t row_bytes, const void* blob,
                            int M, int64_t N, int64_t K, float* y, hipStream_t s) {
    TileArgs a{static_cast<const uint8_t*>(act), row_bytes, static_cast<const uint8_t*>(blob), M, N, K, y};
    if (fmt == kNV) return comp ? launch_tile_t<kNV, true>(a, s) : launch_tile_t<kNV, false>(a, s);
    return comp ? launch_tile_t<kMX, true>(a, s) : launch_tile_t<kMX, false>(a, s);
}

}  // namespace rsfp4
