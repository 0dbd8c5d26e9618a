// gemm_tile.hip -- block-scaled FP4 linear for wide activation operands
// (B > 32 tile rows: prefill-like M, or many decode rows), on the gfx950
// matrix cores.
//
// Same operation as the narrow-M kernel (ResServe, arXiv 2611.08713, Section
// 4.2 Eq. 1 and Section 4.3 Eq. 2: Z = [X^; R^] W^T with the Fold
// Y_j = Z_j + Z_{M+j}), but here the product is dense enough to be bound by the
// matrix cores, so it is tiled in two dimensions.  A workgroup of 4 waves owns
// TB = 16*RTW activation tile rows x TN = 64*CTW output channels:
//   * weights: each wave owns CTW 16-channel groups and streams their packed
//     fragments straight from HBM into a register ring of 4 (NVFP4) or 8
//     (MXFP4) steps (the packed layout puts one MFMA operand in 1 KB of
//     consecutive bytes), loading each fragment exactly once per workgroup,
//     three or seven steps ahead of use, and the block scales once per quad;
//   * activations: shared by all four waves, so they are staged through LDS
//     (double-buffered, global loads one stage ahead).  MXFP4 keeps the FP4
//     codes there (the scaled MFMA consumes them with their E8M0 scales);
//     NVFP4 dequantizes each element once per workgroup to f16 (e * S_b,
//     exact) while writing the stage, so the waves read ready MFMA operands;
//   * MXFP4 multiplies on v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4 with
//     both operands' E8M0 scales); NVFP4 dequantizes weight fragments to f16
//     in registers and uses v_mfma_f32_16x16x32_f16; tensor scales enter the
//     Fold.
// Every global load is unconditional (out-of-range reads return zeros) and
// the per-step address parts are uniform, so the compiler's memory-counter
// waits stay exact and the per-lane address work is done once.
// Tile rows interleave base and residue rows (2m = q(x) row m, 2m+1 = q(r) row
// m), so every accumulator lane holds complete pairs and the Fold is a
// thread-local add before the only store.
//
// Workgroups are mapped to tiles per XCD: XCD x (= workgroup id mod 8) runs a
// contiguous range of tiles ordered row-tile fastest, so the row tiles that
// share a weight tile run together on one XCD and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.h"
#include "fp4_frag.h"
#include "kernels.h"
#include "layout.h"

namespace rsfp4 {

namespace {

constexpr int kXcds = 8;
constexpr uint32_t kOob = 0x80000000u;     // voffset of a lane whose data is outside the operand

// FP4 x FP4 scaled MFMA; oa / ob select the scale byte inside sa / sb.  The
// selectors must be literal constants, hence the switches (they fold away
// once the calling loops are unrolled).
template <int OA>
__device__ __forceinline__ floatx4 mfma_fp4_oa(intx8 a, intx8 b, floatx4 c, int sa, int ob, int sb) {
    switch (ob) {
        case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, 0, sb);
        case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, 1, sb);
        case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, 2, sb);
        default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OA, sa, 3, sb);
    }
}
__device__ __forceinline__ floatx4 mfma_fp4(intx8 a, intx8 b, floatx4 c, int oa, int sa, int ob, int sb) {
    switch (oa) {
        case 0: return mfma_fp4_oa<0>(a, b, c, sa, ob, sb);
        case 1: return mfma_fp4_oa<1>(a, b, c, sa, ob, sb);
        case 2: return mfma_fp4_oa<2>(a, b, c, sa, ob, sb);
        default: return mfma_fp4_oa<3>(a, b, c, sa, ob, sb);
    }
}

// Buffer resource over bytes [off, bytes) of `base`: uniform per-step offsets
// move the base (scalar arithmetic) rather than entering the range-checked
// per-lane offset, so a lane past the end of the operand reads zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const uint8_t* base, int64_t off, int64_t bytes) {
    const int64_t left = bytes - off;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), (short)0, (int)(left > 0 ? left : 0),
                                             kRsrcWord3);
}

struct TileArgs {
    const uint8_t* act;
    int64_t row_bytes;
    const uint8_t* blob;
    int M;
    int64_t N;
    int64_t K;
    void* y;            // fp32 or (out_bf16) bf16 output
    int row_tiles;      // ceil(B / TB)
    int64_t tiles;      // row_tiles * ceil(N / TN)
    int64_t per_xcd;    // ceil(tiles / 8)
    int out_bf16;       // store y as bf16 (round to nearest even)
};

// LDS layout of one activation stage.
//   MXFP4 (2 steps): codes [st][tile][lane] 16 B in fragment order (slot
//   swizzled, see a_slot), then scales [st][lane][tile] 1 B, so that one
//   8-byte read gives a lane the scales of all its row tiles.
//   NVFP4 (1 step): f16 fragments [u][tile][lane] 16 B, u = the 32-element
//   sub-step of the f16 MFMA (slot swizzled, see h_slot).
template <int FMT, int TB>
struct AStage {
    static constexpr int kSteps = FMT == kNV ? 1 : 2;
    static constexpr int kScales = 2 * TB * 64;                       // MXFP4 only
    static constexpr int kBytes = FMT == kNV ? TB * 256 : 2 * TB * 64 + 2 * TB * 4;
};

// 16-byte slot of (row i of a 16-row tile, k-group g) in a 1 KB fragment block.
// The XOR spreads the slots written together over distinct bank groups and
// keeps the reads of 8 consecutive lanes (consecutive rows, one group)
// conflict-free.
__device__ __forceinline__ int a_slot(int i, int g, int st) { return g * 16 + (i ^ (g + 4 * st)); }
__device__ __forceinline__ int h_slot(int i, int g) { return g * 16 + (i ^ (2 * g)); }

template <int FMT, bool COMP, int RTW, int CTW, int RD, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_tile_kernel(TileArgs p) {
    constexpr int TB = 16 * RTW;                  // activation tile rows per workgroup
    constexpr int GPT = 4 * CTW;                  // 16-channel groups per workgroup
    constexpr int SA = AStage<FMT, TB>::kSteps;   // steps per activation stage
    constexpr int kStage = AStage<FMT, TB>::kBytes;
    constexpr int SB = FMT == kNV ? 2 : 1;        // blob scale bytes per lane and step
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // tile of this workgroup (XCD-grouped, row tiles fastest)
    const int64_t L_id = blockIdx.x;
    const int64_t tile = (L_id % kXcds) * p.per_xcd + L_id / kXcds;
    if (tile >= p.tiles) return;                  // uniform: whole workgroup idle
    const int rtile = (int)(tile % p.row_tiles);
    const int64_t ctile = tile / p.row_tiles;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);   // uniform: keeps weight descriptors scalar
    const int g = lane >> 4, i = lane & 15;
    const int64_t G = num_groups(p.N);
    const int64_t GB = group_bytes(FMT, p.K);
    const int64_t QB = quad_bytes(FMT);
    const int nq = (int)((num_steps(p.K) + kQuadSteps - 1) / kQuadSteps);
    const int nq2 = (nq + 1) & ~1;                // quads processed (even: loop unrolled by two)
    const uint32_t scale_base = (uint32_t)(kActHead + p.K / 2);
    const int B = COMP ? 2 * p.M : p.M;
    const int64_t act_bytes = (int64_t)B * p.row_bytes;

    // this wave's weight groups
    const int64_t cw = ctile * GPT + wave * CTW;
    const int64_t live = G - cw < 0 ? 0 : (G - cw < CTW ? G - cw : CTW);
    const uint8_t* wbase = p.blob + kWHeader + (live > 0 ? cw : 0) * GB;
    const int64_t wbytes = live * GB;

    auto act_record = [&](int row) -> uint32_t {  // tile row -> record offset, or kOob
        const int R = TB * rtile + row;
        if (COMP) {
            const int m = R >> 1;
            return m < p.M ? (uint32_t)(((R & 1) ? p.M + m : m) * p.row_bytes) : kOob;
        }
        return R < p.M ? (uint32_t)(R * p.row_bytes) : kOob;
    };

    // ---- activation staging: fixed per-lane parts ----
    // NVFP4: TB rows x 4 k-groups of one step, one 16 B chunk each, plus the
    //        chunk's two block-scale bytes.
    // MXFP4: TB rows x 2 steps x 4 k-groups, then (row, step) scale words.
    constexpr int kACh = FMT == kNV ? TB * 4 / 256 : TB * 8 / 256;
    constexpr int kASc = FMT == kNV ? 0 : TB * 2 / 256;
    uint32_t a_vo[kACh];        // code voffset (kOob for rows outside the operand)
    uint32_t a_so[kACh];        // scale voffset (NVFP4)
    int a_k[kACh];              // k of the chunk inside its stage
    int a_lds[kACh];            // LDS offset of the chunk (first u for NVFP4)
#pragma unroll
    for (int j = 0; j < kACh; ++j) {
        const int c = 256 * j + t;
        if (FMT == kNV) {
            const int row = c >> 2, gg = c & 3;
            const uint32_t rec = act_record(row);
            a_vo[j] = rec == kOob ? kOob : rec + (uint32_t)(kActHead + 16 * gg);
            a_so[j] = rec == kOob ? kOob : rec + scale_base + (uint32_t)(2 * gg);
            a_k[j] = 32 * gg;
            a_lds[j] = ((row >> 4) * 64 + h_slot(row & 15, gg)) * 16;
        } else {
            const int row = c >> 3, st = (c >> 2) & 1, gg = c & 3;
            const uint32_t rec = act_record(row);
            a_vo[j] = rec == kOob ? kOob : rec + (uint32_t)(kActHead + 64 * st + 16 * gg);
            a_so[j] = 0;
            a_k[j] = 128 * st + 32 * gg;
            a_lds[j] = ((st * (TB / 16) + (row >> 4)) * 64 + a_slot(row & 15, gg, st)) * 16;
        }
    }
    uint32_t as_vo[kASc > 0 ? kASc : 1];
    int as_lds[kASc > 0 ? kASc : 1];       // LDS byte of (row, step, group 0); group g adds 16*RTW*g
#pragma unroll
    for (int j = 0; j < kASc; ++j) {
        const int item = 256 * j + t;
        const int row = item >> 1, st = item & 1;
        const uint32_t rec = act_record(row);
        as_vo[j] = rec == kOob ? kOob : rec + scale_base + (uint32_t)(4 * st);
        as_lds[j] = AStage<FMT, TB>::kScales + (st * 64 + (row & 15)) * RTW + (row >> 4);
    }

    struct AReg {               // one activation stage on its way to LDS
        uint4 c[kACh];
        uint32_t s[kACh > kASc ? kACh : kASc];
    };

    auto load_a = [&](int stg, AReg& R) {
        const int64_t k0 = (int64_t)stg * SA * 128;             // first k of the stage
        const __amdgpu_buffer_rsrc_t rc = rsrc_at(p.act, k0 / 2, act_bytes);
        const __amdgpu_buffer_rsrc_t rs = rsrc_at(p.act, k0 / (FMT == kNV ? 16 : 32), act_bytes);
#pragma unroll
        for (int j = 0; j < kACh; ++j) {
            // chunks past K (a partial last step) read zeros
            const bool kin = k0 + a_k[j] < p.K;
            R.c[j] = ld128(rc, kin ? a_vo[j] : kOob);
            if (FMT == kNV) R.s[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, kin ? a_so[j] : kOob, 0, 0);
        }
        if (FMT == kMX) {
#pragma unroll
            for (int j = 0; j < kASc; ++j) R.s[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, as_vo[j], 0, 0);
        }
    };

    auto store_a = [&](const AReg& R, int buf, int stg) {
        uint8_t* base = lds + buf * kStage;
        if (FMT == kNV) {
#pragma unroll
            for (int j = 0; j < kACh; ++j) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const half8 h = dequant8(word(R.c[j], u), scale_h((R.s[j] >> (u < 2 ? 0 : 8)) & 0xFFu));
                    *reinterpret_cast<half8*>(base + u * (TB / 16) * 1024 + a_lds[j]) = h;
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kACh; ++j) *reinterpret_cast<uint4*>(base + a_lds[j]) = R.c[j];
#pragma unroll
            for (int j = 0; j < kASc; ++j) {
                // scale bytes of k-groups past K hold whatever followed the
                // record's scales (their codes read as zero): write 0 instead,
                // since an E8M0 0xFF would be NaN
                const int st = (256 * j + t) & 1;
                const int64_t kleft = p.K - ((int64_t)stg * SA + st) * 128;
                const int nb = kleft >= 128 ? 4 : (kleft <= 0 ? 0 : (int)(kleft / 32));
#pragma unroll
                for (int gg = 0; gg < 4; ++gg)
                    base[as_lds[j] + 16 * RTW * gg] = gg < nb ? (uint8_t)(R.s[j] >> (8 * gg)) : (uint8_t)0;
            }
        }
    };

    // ---- weight streaming: ring of 4 steps, scale words per quad ----
    uint32_t b_vo[CTW], bs_vo[CTW];
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
        b_vo[ct] = (uint32_t)(ct * GB) + 16u * lane;
        bs_vo[ct] = (uint32_t)(ct * GB) + 4096u + (uint32_t)(lane * 4 * SB);
    }
    static_assert(RD == 4 || RD == 8, "ring depth divides the 8-step loop body");
    uint4 ring[RD][CTW];
    u32x2 sw[2][CTW];           // NVFP4: 8 scale bytes per quad; MXFP4: 4 (word 0)

    auto load_b = [&](int s, int slot) {    // step s into ring slot (zeros past the last quad)
        const __amdgpu_buffer_rsrc_t r = rsrc_at(wbase, (int64_t)(s / kQuadSteps) * QB + (s % kQuadSteps) * 1024, wbytes);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) ring[slot][ct] = ld128(r, b_vo[ct]);
    };
    auto load_sw = [&](int q, int slot) {   // scale words of quad q
        const __amdgpu_buffer_rsrc_t r = rsrc_at(wbase, (int64_t)q * QB, wbytes);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            if (FMT == kNV)
                sw[slot][ct] = __builtin_amdgcn_raw_buffer_load_b64(r, bs_vo[ct], 0, 0);
            else
                sw[slot][ct] = u32x2{__builtin_amdgcn_raw_buffer_load_b32(r, bs_vo[ct], 0, 0), 0u};
        }
    };

    floatx4 acc[RTW][CTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) acc[rt][ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // one 128-element step: activations from LDS stage buffer `buf` (step st
    // of that stage), weights from ring slot `slot`, scale bytes of quad step
    // u.  MXFP4: a step's LDS reads are all issued before its MFMAs
    // (scheduling groups), so the LDS latency is exposed once per step, not
    // per tile.  NVFP4 pins its reads and the weight dequantization ahead of
    // the MFMAs with a plain scheduling barrier (scheduling groups there make
    // the compiler's group solver take unbounded time).
    auto compute = [&](int buf, int st, int slot, int qs, int u) {
        const uint8_t* base = lds + buf * kStage;
        if (FMT == kNV) {
#pragma unroll
            for (int u4 = 0; u4 < 4; ++u4) {
                half8 ah[RTW], bh[CTW];
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
                    ah[rt] = *reinterpret_cast<const half8*>(base + ((u4 * (TB / 16) + rt) * 64 + h_slot(i, g)) * 16);
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) {
                    const uint32_t sword = u < 2 ? sw[qs][ct][0] : sw[qs][ct][1];
                    const uint32_t sb = (sword >> (16 * (u & 1) + (u4 < 2 ? 0 : 8))) & 0xFFu;
                    bh[ct] = dequant8(word(ring[slot][ct], u4), scale_h(sb));
                }
                // reads and dequantization stay ahead of the MFMAs that use them
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct)
                        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bh[ct], acc[rt][ct], 0, 0, 0);
            }
        } else {
            uint4 a[RTW];
            uint32_t as[(RTW + 3) / 4];
            static_assert(RTW % 4 == 0, "scale words hold four row tiles");
            if (RTW == 8) {
                const u32x2 w2 = *reinterpret_cast<const u32x2*>(base + AStage<FMT, TB>::kScales + (st * 64 + lane) * RTW);
                as[0] = w2[0];
                as[1] = w2[1];
            } else {
                as[0] = *reinterpret_cast<const uint32_t*>(base + AStage<FMT, TB>::kScales + (st * 64 + lane) * RTW);
            }
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt)
                a[rt] = *reinterpret_cast<const uint4*>(base + ((st * (TB / 16) + rt) * 64 + a_slot(i, g, st)) * 16);
#pragma unroll
            for (int rt = 0; rt < RTW; ++rt) {
                const intx8 av = {(int)a[rt].x, (int)a[rt].y, (int)a[rt].z, (int)a[rt].w, 0, 0, 0, 0};
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) {
                    const uint4 b = ring[slot][ct];
                    const intx8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
                    // op_sel picks the scale byte: row tile rt of the A word,
                    // quad step u of the B word
                    acc[rt][ct] = mfma_fp4(av, bv, acc[rt][ct], rt & 3, (int)as[rt >> 2], u, (int)sw[qs][ct][0]);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, RTW + 1, 0);          // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, RTW * CTW, 0);        // MFMAs
        }
    };

    // ---- pipeline ----
    // Activation stages go global -> registers -> LDS with two register sets:
    // a set is loaded two stages before it is written to LDS, so its loads have
    // two stages of compute to land in.
    AReg RA0, RA1;
    load_a(0, RA0);
    load_a(1, RA1);
    load_sw(0, 0);
    load_b(0, 0);
    store_a(RA0, 0, 0);
    load_a(2, RA0);
#pragma unroll
    for (int r = 1; r < RD - 1; ++r)   // the prologue ends with weight loads, as
        load_b(r, r);                  // every loop step does, so the loop's waits stay partial
    __syncthreads();
    // Two quads (8 steps) per iteration so that every ring, scale-word, LDS
    // buffer and register-set index is static (an iteration starts at an even
    // stage).  Step s: its activation stage is s / SA, in LDS buffer
    // (s / SA) % 2; at the first step of stage t, stage t+1 (loaded two stages
    // earlier) is written to the other buffer, whose last reader was stage
    // t-1, and stage t+3 is loaded into the freed set; a barrier closes each
    // stage.
    for (int q = 0; q < nq2; q += 2) {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            const int s = 4 * q + v;
            const int qs = v >> 2, u = v & 3;
            if (u == 0) load_sw(q + qs + 1, qs ^ 1);
            const int stg = s / SA;
            const int st = v % SA;
            const int par = (v / SA) & 1;          // parity of stg
            if (st == 0) {
                AReg& R = par ? RA0 : RA1;         // holds stage stg+1
                store_a(R, par ^ 1, stg + 1);
                load_a(stg + 3, R);
            }
            load_b(s + RD - 1, (v + RD - 1) % RD);
            // keep the global loads where they are in program order (the
            // scheduler would otherwise sink some next to their distant use)
            __builtin_amdgcn_sched_barrier(0x070E);
            compute(par, st, v % RD, qs, u);
            if (st == SA - 1) __syncthreads();
        }
    }

    // ---- Fold + store: lane holds tile rows 16rt + 4g + r of channel 16(cw+ct) + i ----
    float s_gw = 1.0f;
    if (FMT == kNV) s_gw = reinterpret_cast<const WHeader*>(p.blob)->s_g;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int64_t n = 16 * (cw + ct) + i;
            if (n >= p.N) continue;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const int R0 = TB * rtile + 16 * rt + 4 * g + 2 * pr;
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
                        store_y(p.y, (int64_t)m * p.N + n, out, p.out_bf16);
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
                            store_y(p.y, (int64_t)m * p.N + n, out, p.out_bf16);
                        }
                    }
                }
            }
        }
    }
}

template <int FMT, bool COMP, int RTW, int CTW, int RD, int OCC>
hipError_t launch_tile_t(TileArgs a, hipStream_t s) {
    constexpr int TB = 16 * RTW, TN = 64 * CTW;
    constexpr int lds = 2 * AStage<FMT, TB>::kBytes;
    auto kern = gemm_tile_kernel<FMT, COMP, RTW, CTW, RD, OCC>;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (attr != hipSuccess) return attr;
    const int B = COMP ? 2 * a.M : a.M;
    a.row_tiles = (B + TB - 1) / TB;
    a.tiles = (int64_t)a.row_tiles * ((a.N + TN - 1) / TN);
    a.per_xcd = (a.tiles + kXcds - 1) / kXcds;
    const int64_t grid = a.per_xcd * kXcds;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, a);
    return hipGetLastError();
}

// Tile configurations (from a sweep on the wide workloads).  NVFP4 steps
// carry four f16 MFMAs per tile: a 128 x 128 tile with a 4-step weight ring at
// two workgroups per CU.  An MXFP4 step is a single FP4 MFMA per tile, so its
// activation fragments are read from LDS four times as often per MFMA; a
// 128 x 256 tile halves that, at one workgroup per CU.
template <int FMT, bool COMP>
hipError_t launch_fmt(const TileArgs& a, hipStream_t s) {
    if (FMT == kNV) return launch_tile_t<FMT, COMP, 8, 2, 4, 2>(a, s);
    return launch_tile_t<FMT, COMP, 8, 4, 4, 1>(a, s);
}

}  // namespace

hipError_t launch_gemm_tile(int fmt, bool comp, const void* act, int64_t row_bytes, const void* blob,
                            int M, int64_t N, int64_t K, void* y, bool out_bf16, hipStream_t s) {
    TileArgs a{static_cast<const uint8_t*>(act), row_bytes, static_cast<const uint8_t*>(blob), M, N, K, y,
               0, 0, 0, out_bf16 ? 1 : 0};
    if (fmt == kNV) return comp ? launch_fmt<kNV, true>(a, s) : launch_fmt<kNV, false>(a, s);
    return comp ? launch_fmt<kMX, true>(a, s) : launch_fmt<kMX, false>(a, s);
}

}  // namespace rsfp4
