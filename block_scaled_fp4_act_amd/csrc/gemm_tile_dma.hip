// gemm_tile_dma.hip -- MXFP4 linear for wide activation operands with both
// operands streamed global -> LDS by the buffer loads' LDS-DMA form.
//
// Same operation as the register-staged tiled kernel (ResServe, arXiv
// 2611.08713, Section 4.2 Eq. 1 and Section 4.3 Eq. 2: Z = [X^; R^] W^T with
// the Fold Y_j = Z_j + Z_{M+j}; MXFP4 blocks of 32 with E8M0 scales, Section
// 2).  Two launches:
//   1. act_tile_kernel rewrites the quantized activation records into the
//      packed-weight layout (groups of 16 rows; per 128-element step 1 KB of
//      codes in MFMA operand order, lane l = 16g + i owning row i, elements
//      32g..32g+31; after every 4 steps the lanes' scale words), the stacked
//      rows interleaved (row 2m = q(x) row m, row 2m+1 = q(r) row m) so that
//      every accumulator lane holds complete pairs for the Fold.  Rows past
//      the operand and elements past K get zero codes and zero scales.  It is
//      a byte permutation of the records: no arithmetic.  A record row holds
//      64 bytes per step, so gathering a 16-row fragment straight from the
//      records costs 16 partial cache lines per 1 KB (measured: 48 against 118
//      GB/s per compute unit for contiguous 1 KB requests); in tiles every
//      fragment of either operand is one contiguous request.
//   2. gemm_tile_mx_dma multiplies the two tiled operands (below).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "codec.h"
#include "fp4_frag.h"
#include "kernels.h"
#include "layout.h"

namespace rsfp4 {

namespace {

constexpr int kXcds = 8;

// ---- 1. activation records -> tiled operand ----
// One thread per 16-byte code chunk or per lane scale word of the output.
template <bool COMP>
__global__ __launch_bounds__(256) void act_tile_kernel(const uint8_t* __restrict__ act, int64_t row_bytes, int M,
                                                       int64_t K, int64_t groups, uint8_t* __restrict__ out) {
    const int64_t nq = num_quads(K);
    const int64_t GB = group_bytes(kMX, K), QB = quad_bytes(kMX);
    const int64_t per_group = nq * (4 * 64 + 64);
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= groups * per_group) return;
    const int64_t grp = item / per_group;
    const int64_t r = item - grp * per_group;
    const int64_t q = r / 320;
    const int w = (int)(r - q * 320);
    const int l = w & 63, g = l >> 4, i = l & 15;
    const int64_t R = 16 * grp + i;                    // stacked operand row
    int64_t rec = -1;
    if (COMP) {
        const int64_t m = R >> 1;
        if (m < M) rec = ((R & 1) ? M + m : m) * row_bytes;
    } else if (R < M) {
        rec = R * row_bytes;
    }
    uint8_t* grp_out = out + grp * GB + q * QB;
    if (w < 256) {                                     // codes: step u of the quad, lane l
        const int u = w >> 6;
        const int64_t k = (4 * q + u) * kStepK + 32 * g;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (rec >= 0 && k < K) v = *reinterpret_cast<const uint4*>(act + rec + kActHead + k / 2);
        *reinterpret_cast<uint4*>(grp_out + u * kStepCodes + 16 * l) = v;
    } else {                                           // lane l's E8M0 bytes of block g, steps 4q..4q+3
        const int64_t sbase = rec + kActHead + K / 2;
        uint32_t word = 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t s = 4 * q + u;
            if (rec >= 0 && s * kStepK + 32 * g < K) word |= (uint32_t)act[sbase + 4 * s + g] << (8 * u);
        }
        *reinterpret_cast<uint32_t*>(grp_out + kQuadSteps * kStepCodes + 4 * l) = word;
    }
}


// NVFP4: one thread per (16-row group, step, lane): the lane's 32 codes and
// their two E4M3 block scales -> four 16-byte f16 fragments e * S_b (exact, the
// values the register-staged kernel forms in LDS; the tensor scale stays out,
// applied in the epilogue), one per 32-element sub-step of the f16 MFMA, at
// group * S * 4 KB + step * 4 KB + u * 1 KB.
template <bool COMP>
__global__ __launch_bounds__(256) void act_tile_f16_kernel(const uint8_t* __restrict__ act, int64_t row_bytes, int M,
                                                           int64_t K, int64_t groups, uint8_t* __restrict__ out) {
    const int64_t S = num_steps(K);
    const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (item >= groups * S * 64) return;
    const int64_t grp = item / (S * 64);
    const int64_t r = item - grp * S * 64;
    const int64_t s = r >> 6;
    const int l = (int)(r & 63), g = l >> 4, i = l & 15;
    const int64_t R = 16 * grp + i;
    int64_t rec = -1;
    if (COMP) {
        const int64_t m = R >> 1;
        if (m < M) rec = ((R & 1) ? M + m : m) * row_bytes;
    } else if (R < M) {
        rec = R * row_bytes;
    }
    const int64_t k = s * kStepK + 32 * g;
    uint4 c = make_uint4(0u, 0u, 0u, 0u);
    uint32_t sc = 0u;
    if (rec >= 0 && k < K) {
        c = *reinterpret_cast<const uint4*>(act + rec + kActHead + k / 2);
        const uint8_t* sp = act + rec + kActHead + K / 2 + k / 16;     // blocks 2g, 2g+1 of the step
        sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
    }
    uint8_t* dst = out + grp * S * 4096 + s * 4096 + 16 * l;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const half8 h = dequant8(word(c, u), scale_h(u < 2 ? (sc & 0xFFu) : (sc >> 8)));
        *reinterpret_cast<half8*>(dst + u * 1024) = h;
    }
}

// ---- 2. the tiled products ----
// Both kernels stream the two tiled operands into a ring of LDS stages with
// the buffer loads' LDS-DMA form (each request: 64 lanes x 16 bytes, one
// contiguous 1 KB fragment) and track them with the vector-memory counter.
// Every step starts with a wait for this wave's requests of its stage (what was
// requested after it stays in flight) and a workgroup barrier fenced for LDS
// only (a workgroup fence would also wait for the later stages' requests); the
// barrier publishes the stage and frees the buffer the previous step read,
// which is refilled right after it.  The matrix cores reach their rate only
// with two waves per SIMD (one wave issuing independent MFMAs back to back
// sustains about 60 % of it), so a workgroup runs 8 waves, or 4 waves with two
// workgroups per compute unit, within 256 registers per wave; the other wave of
// a SIMD hides each wave's LDS latency and barrier waits.

// One request of 64 lanes: each lane's 16 (4) bytes at voffset vo of r land in
// LDS at dst + 16 * lane (4 * lane); dst is uniform.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t vo) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, vo, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t vo) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4, vo, 0, 0, 0);
}

// s_waitcnt bounding only the vector-memory counter (gfx9 field layout:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// This wave's LDS reads done, then the workgroup barrier (no memory fence).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Buffer resource over bytes [off, bytes) of base (zeros past the end).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const uint8_t* base, int64_t off, int64_t bytes) {
    const int64_t left = bytes - off;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + off), (short)0, (int)(left > 0 ? left : 0), kRsrcWord3);
}

// FP4 x FP4 scaled MFMA, both scale bytes selected by quad step U.
template <int U>
__device__ __forceinline__ floatx4 mfma_fp4_u(const uint4& a, const uint4& b, floatx4 c, uint32_t sa, uint32_t sb) {
    const intx8 av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const intx8 bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, U, (int)sa, U, (int)sb);
}

// Tile of the workgroup: per XCD a contiguous range of tiles, row tiles
// fastest, so the row tiles that share a weight tile run together on one L2.
struct TileGrid {
    int row_tiles;
    int64_t tiles;
    int64_t per_xcd;
};
__device__ __forceinline__ bool tile_of(const TileGrid& t, int* rtile, int64_t* ctile) {
    const int64_t L_id = blockIdx.x;
    const int64_t tile = (L_id % kXcds) * t.per_xcd + L_id / kXcds;
    if (tile >= t.tiles) return false;
    *rtile = (int)(tile % t.row_tiles);
    *ctile = tile / t.row_tiles;
    return true;
}
inline TileGrid tile_grid(int64_t B, int64_t N, int TM, int TN) {
    TileGrid t;
    t.row_tiles = (int)((B + TM - 1) / TM);
    t.tiles = (int64_t)t.row_tiles * ((num_groups(N) + TN / 16 - 1) / (TN / 16));
    t.per_xcd = (t.tiles + kXcds - 1) / kXcds;
    return t;
}

// ---- MXFP4: both operands in the packed-weight layout ----
// WR x WC waves; a wave owns RTW x CTW output tiles of 16 x 16, the workgroup
// TM = 16*RTW*WR rows x TN = 16*CTW*WC channels.  A stage holds one step's
// fragments of both operands; 4 stages rotate (stage s+4 requested in step s,
// after its barrier), and a 2-slot ring holds the scale words of the current
// and the next quad (requested in a quad's second step, read in its last).  Each step's MFMAs
// are v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4 with both operands' E8M0
// scales, the quad step selecting the scale byte), summed over the steps in
// order, as the register-staged kernel does: the result is bit-identical.
template <int RTW, int CTW, int WR, int WC>
struct MxTile {
    static constexpr int NW = WR * WC;
    static constexpr int TM = 16 * RTW * WR, TN = 16 * CTW * WC;
    static constexpr int AFR = TM / 16, BFR = TN / 16;     // fragments per step
    static constexpr int B_OFF = AFR * 1024;
    static constexpr int STAGE = (AFR + BFR) * 1024;
    static constexpr int SQ = (AFR + BFR) * 256;           // scale words of one quad, both operands
    static constexpr int DA = AFR / NW, DB = BFR / NW;     // per-wave requests of one stage
    static constexpr int D = DA + DB;
    static constexpr int DS = DA + DB;                     // per-wave scale requests of one quad
    static_assert(AFR % NW == 0 && BFR % NW == 0, "fragments split evenly over the waves");
    static_assert(4 * STAGE + 2 * SQ <= 160 * 1024, "the ring fits in LDS");
};

struct DmaArgs {
    const uint8_t* at;   // tiled activation operand (act_tile_kernel)
    const uint8_t* blob; // packed weights
    int M;
    int64_t N;
    int64_t K;
    void* y;
    int out_bf16;
    TileGrid grid;
};

template <bool COMP, int RTW, int CTW, int WR, int WC, int OCC>
__global__ __launch_bounds__(64 * WR * WC, OCC) void gemm_tile_mx_dma(DmaArgs p) {
    using T = MxTile<RTW, CTW, WR, WC>;
    __shared__ __attribute__((aligned(16))) uint8_t st0[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st3[T::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t sq0[T::SQ];
    __shared__ __attribute__((aligned(16))) uint8_t sq1[T::SQ];

    int rtile;
    int64_t ctile;
    if (!tile_of(p.grid, &rtile, &ctile)) return;       // uniform: the whole workgroup

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    const int wr = wave / WC, wc = wave % WC;
    const int64_t GB = group_bytes(kMX, p.K);
    const int64_t QB = quad_bytes(kMX);
    const int S = (int)num_steps(p.K);
    const int nq2 = (((S + kQuadSteps - 1) / kQuadSteps) + 1) & ~1;   // quads, rounded to even
    const int B = COMP ? 2 * p.M : p.M;

    // operand tiles: groups [a0, a0 + AFR) of the tiled activations and
    // [b0, b0 + BFR) of the weights (ranges clipped: groups past the end read zeros)
    const int64_t GA = (B + 15) / 16, GW = num_groups(p.N);
    const int64_t a0 = (int64_t)rtile * T::AFR, b0 = ctile * T::BFR;
    const uint8_t* abase = p.at + a0 * GB;
    const uint8_t* bbase = p.blob + kWHeader + b0 * GB;
    const int64_t abytes = (GA - a0 < T::AFR ? GA - a0 : T::AFR) * GB;
    const int64_t bbytes = (GW - b0 < T::BFR ? GW - b0 : T::BFR) * GB;

    // per-lane request offsets inside a tile: fragment j of this wave is group wave + NW*j
    uint32_t a_vo[T::DA], b_vo[T::DB], as_vo[T::DA], bs_vo[T::DB];
#pragma unroll
    for (int j = 0; j < T::DA; ++j) {
        a_vo[j] = (uint32_t)((wave + T::NW * j) * GB) + 16u * lane;
        as_vo[j] = (uint32_t)((wave + T::NW * j) * GB) + kQuadSteps * kStepCodes + 4u * lane;
    }
#pragma unroll
    for (int j = 0; j < T::DB; ++j) {
        b_vo[j] = (uint32_t)((wave + T::NW * j) * GB) + 16u * lane;
        bs_vo[j] = (uint32_t)((wave + T::NW * j) * GB) + kQuadSteps * kStepCodes + 4u * lane;
    }

    auto stage_buf = [&](int b) -> uint8_t* { return b == 0 ? st0 : (b == 1 ? st1 : (b == 2 ? st2 : st3)); };

    auto dma_stage = [&](int s, int b) {      // step s's fragments into stage buffer b
        uint8_t* dst = stage_buf(b);
        const int64_t off = (int64_t)(s / kQuadSteps) * QB + (s % kQuadSteps) * kStepCodes;
        const __amdgpu_buffer_rsrc_t ra = rsrc_at(abase, off, abytes);
        const __amdgpu_buffer_rsrc_t rb = rsrc_at(bbase, off, bbytes);
#pragma unroll
        for (int j = 0; j < T::DA; ++j) dma16(ra, dst + (wave + T::NW * j) * 1024, a_vo[j]);
#pragma unroll
        for (int j = 0; j < T::DB; ++j) dma16(rb, dst + T::B_OFF + (wave + T::NW * j) * 1024, b_vo[j]);
    };
    auto dma_scales = [&](int q, int slot) {  // quad q's scale words into ring slot
        uint8_t* dst = slot ? sq1 : sq0;
        const __amdgpu_buffer_rsrc_t ra = rsrc_at(abase, (int64_t)q * QB, abytes);
        const __amdgpu_buffer_rsrc_t rb = rsrc_at(bbase, (int64_t)q * QB, bbytes);
#pragma unroll
        for (int j = 0; j < T::DA; ++j) dma4(ra, dst + (wave + T::NW * j) * 256, as_vo[j]);
#pragma unroll
        for (int j = 0; j < T::DB; ++j) dma4(rb, dst + (T::AFR + wave + T::NW * j) * 256, bs_vo[j]);
    };

    struct Frag {
        uint4 a[RTW];
        uint4 b[CTW];
    };
    struct Scales {
        uint32_t a[RTW];
        uint32_t b[CTW];
    };
    Frag F0, F1;
    Scales Q0, Q1;
    floatx4 acc[RTW][CTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) acc[rt][ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    auto read_stage = [&](int b, Frag& F) {
        const uint8_t* src = stage_buf(b);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
            F.a[rt] = *reinterpret_cast<const uint4*>(src + (wr * RTW + rt) * 1024 + 16 * lane);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            F.b[ct] = *reinterpret_cast<const uint4*>(src + T::B_OFF + (wc * CTW + ct) * 1024 + 16 * lane);
    };
    auto read_scales = [&](int slot, Scales& Q) {
        const uint8_t* sq = slot ? sq1 : sq0;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
            Q.a[rt] = *reinterpret_cast<const uint32_t*>(sq + (wr * RTW + rt) * 256 + 4 * lane);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            Q.b[ct] = *reinterpret_cast<const uint32_t*>(sq + (T::AFR + wc * CTW + ct) * 256 + 4 * lane);
    };
    auto mfmas = [&](const Frag& F, const Scales& Q, auto u_tag, int rt0, int rt1) {
        constexpr int U = decltype(u_tag)::value;
#pragma unroll
        for (int rt = rt0; rt < rt1; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
                acc[rt][ct] = mfma_fp4_u<U>(F.a[rt], F.b[ct], acc[rt][ct], Q.a[rt], Q.b[ct]);
    };

    // Step s runs the first half of its MFMAs on fragments read during step
    // s-1, waits for stage s+1 and passes the barrier (all waves' reads of
    // stage s are then done), requests stage s+4 into stage s's buffer, reads
    // stage s+1's fragments into the other register set and runs its second
    // half: the reads overlap MFMAs instead of following the barrier.
    // Requests in program order: prologue [scales q0, stages 0..3]; step s,
    // after its barrier: [scales of quad q+1 if s % 4 == 1], stage s+4.  The
    // wait for stage s+1 (requested in step s-3, or the prologue) leaves in
    // flight stages s+2 and s+3, and at s % 4 == 2 the next quad's scales
    // (requested in step s-1); at s % 4 == 3 those scales are read after the
    // barrier, so the wait covers them too.
    dma_scales(0, 0);
    dma_stage(0, 0);
    dma_stage(1, 1);
    dma_stage(2, 2);
    dma_stage(3, 3);
    wait_vm<3 * T::D>();
    lds_barrier();
    read_stage(0, F0);
    read_scales(0, Q0);
    for (int q = 0; q < nq2; q += 2) {
        auto step = [&](auto v_tag) {
            constexpr int v = decltype(v_tag)::value;       // step of the two-quad body
            constexpr int u = v & 3, qp = v >> 2;
            const int s = 4 * q + v;
            Frag& Fc = (v & 1) ? F1 : F0;
            Frag& Fn = (v & 1) ? F0 : F1;
            Scales& Qc = qp ? Q1 : Q0;
            const std::integral_constant<int, u> ut;
            const bool live = s < S;                       // padding steps of the last quad: no MFMAs
            __builtin_amdgcn_sched_barrier(0);
            if (live) mfmas(Fc, Qc, ut, 0, RTW / 2);
            if (u == 2) wait_vm<2 * T::D + T::DS>();
            else wait_vm<2 * T::D>();
            lds_barrier();
            if (u == 1) dma_scales(q + qp + 1, qp ^ 1);
            dma_stage(s + 4, v & 3);
            read_stage((v + 1) & 3, Fn);
            if (u == 3) read_scales(qp ^ 1, qp ? Q0 : Q1);
            if (live) mfmas(Fc, Qc, ut, RTW / 2, RTW);
        };
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
        step(std::integral_constant<int, 2>());
        step(std::integral_constant<int, 3>());
        step(std::integral_constant<int, 4>());
        step(std::integral_constant<int, 5>());
        step(std::integral_constant<int, 6>());
        step(std::integral_constant<int, 7>());
    }
    // the requests of the stages past the end land before the LDS is released
    wait_vm<0>();

    // ---- Fold + store: lane holds operand rows 16f + 4g + r of channel 16(group) + i ----
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int64_t n = 16 * (b0 + wc * CTW + ct) + i;
            if (n >= p.N) continue;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const int R0 = T::TM * rtile + 16 * (wr * RTW + rt) + 4 * g + 2 * pr;
                const float v0 = acc[rt][ct][2 * pr], v1 = acc[rt][ct][2 * pr + 1];
                if (COMP) {
                    const int m = R0 >> 1;
                    if (m < p.M) store_y(p.y, (int64_t)m * p.N + n, v0 + v1, p.out_bf16);
                } else {
                    if (R0 < p.M) store_y(p.y, (int64_t)R0 * p.N + n, v0, p.out_bf16);
                    if (R0 + 1 < p.M) store_y(p.y, (int64_t)(R0 + 1) * p.N + n, v1, p.out_bf16);
                }
            }
        }
    }
}

template <bool COMP, int RTW, int CTW, int WR, int WC, int OCC>
hipError_t launch_mx_dma(DmaArgs a, hipStream_t s) {
    using T = MxTile<RTW, CTW, WR, WC>;
    a.grid = tile_grid(COMP ? 2 * (int64_t)a.M : a.M, a.N, T::TM, T::TN);
    auto kern = gemm_tile_mx_dma<COMP, RTW, CTW, WR, WC, OCC>;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.grid.per_xcd * kXcds)), dim3(64 * T::NW), 0, s, a);
    return hipGetLastError();
}

// Tile choice: the largest tile whose tile count still gives three quarters
// of the compute units a tile; 256-row tiles only above 128 operand rows
// (below, half of each tile would be empty).  256 x 256 and 256 x 128 tiles run
// 8 waves (one workgroup per compute unit), 128 x 128 tiles 4 waves with two
// workgroups per compute unit.
template <bool COMP>
hipError_t launch_mx_tiles(const DmaArgs& a, int num_cus, hipStream_t s) {
    const int64_t B = COMP ? 2 * (int64_t)a.M : a.M;
    const int64_t G = num_groups(a.N);
    const int64_t want = (3 * (int64_t)num_cus + 3) / 4;
    if ((B + 255) / 256 * ((G + 15) / 16) >= want) return launch_mx_dma<COMP, 8, 4, 2, 4, 1>(a, s);
    if (B > 128 && (B + 255) / 256 * ((G + 7) / 8) >= want) return launch_mx_dma<COMP, 8, 2, 2, 4, 1>(a, s);
    return launch_mx_dma<COMP, 4, 4, 2, 2, 2>(a, s);
}


// ---- NVFP4: f16 activation fragments (DMA) x weights from a register ring ----
// The register-staged kernel's structure (each wave all the workgroup's rows
// and its own 2 groups of 16 channels, whose weight fragments it streams into
// a register ring 3 steps ahead and dequantizes to f16 at use, the scale words
// a quad ahead), with the activation staging replaced: the f16 fragments of
// each step stream into LDS stages by DMA instead of passing through
// registers, a dequantization and LDS stores in every workgroup.  Tiles of 64
// or 128 rows, 4 or 8 waves (128 or 256 channels) sharing each stage, and K
// optionally split across workgroups (see nv_tile_rows, nv_waves and
// nv_tile_split below).  Same f16 operands and MFMA order as that kernel:
// bit-identical results (unsplit).
struct NvArgs {
    const uint8_t* at;     // f16 activation fragments (act_tile_f16_kernel)
    const uint8_t* act;    // the activation records (per-row tensor scales)
    int64_t row_bytes;
    const uint8_t* blob;
    int M;
    int64_t N;
    int64_t K;
    void* y;
    int out_bf16;
    TileGrid grid;      // over tiles x ks workgroups
    int ks;             // K slices (1: no split)
    int sl;             // steps per slice (a multiple of 8; the last slice may be shorter)
    int* cnt;           // ks > 1: one zeroed counter per tile and wave
    float* part;        // ks > 1: partial sums, per tile, wave and slice
};

// NW waves, each with RTW 16-row tiles (the workgroup's rows, every wave) x
// CTW 16-channel groups; NS activation stages in LDS (2 or 4: the activations
// of step s are requested NS - 1 steps ahead)
template <bool COMP, int RTW, int CTW, int NS, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void gemm_tile_nv_dma(NvArgs p) {
    static_assert(NS == 2 || NS == 4, "two or four activation stages");
    static_assert((4 * RTW) % NW == 0, "a stage's 1 KB blocks divide among the waves");
    constexpr int RD = 4;                             // weight ring depth (steps)
    constexpr int TM = 16 * RTW, GPT = NW * CTW;      // workgroup rows, channel groups
    constexpr int STAGE = RTW * 4096;                 // one step of TM rows as f16: [u4][rt] blocks of 1 KB
    constexpr int DA = 4 * RTW / NW;                  // per-wave requests of one stage
    __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[NS == 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st3[NS == 4 ? STAGE : 16];

    // workgroup -> (tile, K slice): per XCD a contiguous range, slices of a
    // tile fastest, then row tiles (which share a weight tile)
    const int64_t L_id = blockIdx.x;
    const int64_t t_id = (L_id % kXcds) * p.grid.per_xcd + L_id / kXcds;
    if (t_id >= p.grid.tiles) return;
    const int split = (int)(t_id % p.ks);
    const int64_t tile = t_id / p.ks;
    const int rtile = (int)(tile % p.grid.row_tiles);
    const int64_t ctile = tile / p.grid.row_tiles;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, i = lane & 15;
    // this workgroup's steps [s_lo, s_lo + S)
    const int S_all = (int)num_steps(p.K);
    const int s_lo = split * p.sl;
    const int S = S_all - s_lo < p.sl ? S_all - s_lo : p.sl;
    const int nq2 = (((S + kQuadSteps - 1) / kQuadSteps) + 1) & ~1;
    const int64_t GB = group_bytes(kNV, p.K), QB = quad_bytes(kNV);
    const int64_t GA = (int64_t)S_all * 4096;         // f16 fragments of one 16-row group
    const int B = COMP ? 2 * p.M : p.M;
    const int64_t NGA = (B + 15) / 16, G = num_groups(p.N);
    const int64_t a0 = (int64_t)rtile * RTW;
    const uint8_t* abase = p.at + a0 * GA + (int64_t)s_lo * 4096;
    const int64_t abytes = (NGA - a0 < RTW ? NGA - a0 : RTW) * GA - (int64_t)s_lo * 4096;
    const int64_t cw = ctile * GPT + wave * CTW;      // this wave's weight groups
    const int64_t live = G - cw < 0 ? 0 : (G - cw < CTW ? G - cw : CTW);
    const int64_t wq0 = (int64_t)(s_lo / kQuadSteps) * QB;   // the slice's first quad
    const uint8_t* wbase = p.blob + kWHeader + (live > 0 ? cw : 0) * GB + wq0;
    const int64_t wbytes = live * GB - wq0;

    // activation request j of this wave: block wave + 4j = (16-row tile rt, sub-step u4)
    uint32_t a_vo[DA];
    int a_dst[DA];
#pragma unroll
    for (int j = 0; j < DA; ++j) {
        const int blk = wave + NW * j, rt = blk >> 2, u4 = blk & 3;
        a_vo[j] = (uint32_t)(rt * GA) + (uint32_t)(u4 * 1024) + 16u * lane;
        a_dst[j] = (u4 * RTW + rt) * 1024;
    }
    uint32_t b_vo[CTW], bs_vo[CTW];
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
        b_vo[ct] = (uint32_t)(ct * GB) + 16u * lane;
        bs_vo[ct] = (uint32_t)(ct * GB) + kQuadSteps * kStepCodes + 8u * lane;
    }
    auto dma_a = [&](int s, uint8_t* dst) {
        const __amdgpu_buffer_rsrc_t r = rsrc_at(abase, (int64_t)s * 4096, abytes);
#pragma unroll
        for (int j = 0; j < DA; ++j) dma16(r, dst + a_dst[j], a_vo[j]);
    };
    uint4 ring[RD][CTW];
    u32x2 sw[2][CTW];
    auto load_b = [&](int s, int slot) {
        const __amdgpu_buffer_rsrc_t r =
            rsrc_at(wbase, (int64_t)(s / kQuadSteps) * QB + (s % kQuadSteps) * kStepCodes, wbytes);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) ring[slot][ct] = ld128(r, b_vo[ct]);
    };
    auto load_sw = [&](int q, int slot) {
        const __amdgpu_buffer_rsrc_t r = rsrc_at(wbase, (int64_t)q * QB, wbytes);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) sw[slot][ct] = __builtin_amdgcn_raw_buffer_load_b64(r, bs_vo[ct], 0, 0);
    };

    floatx4 acc[RTW][CTW];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) acc[rt][ct] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // the stage of step s (s % NS, a compile-time index: the LDS-DMA writes
    // then go to distinct arrays, which keeps the compiler's waits exact)
    auto stage = [&](auto k_tag) -> uint8_t* {
        constexpr int k = decltype(k_tag)::value % NS;
        if constexpr (k == 0) return st0;
        else if constexpr (k == 1) return st1;
        else if constexpr (k == 2) return st2;
        else return st3;
    };
    if constexpr (NS == 2) {
        load_sw(0, 0);
#pragma unroll
        for (int r = 0; r < RD - 2; ++r) load_b(r, r);
        dma_a(0, st0);
        load_b(RD - 2, RD - 2);
    } else {
        // steps 0..2 requested as steps -3..-1 would (activations, then
        // weights), the first quad's scales before them
        load_sw(0, 0);
        dma_a(0, st0);
        load_b(0, 0);
        dma_a(1, st1);
        load_b(1, 1);
        dma_a(2, st2);
        load_b(2, 2);
    }
    for (int q = 0; q < nq2; q += 2) {
        auto step = [&](auto v_tag) {
            constexpr int v = decltype(v_tag)::value;   // step of the two-quad body
            constexpr int u = v & 3, qs = v >> 2;
            const int s = 4 * q + v;
            if constexpr (NS == 2) {
                // Requests in program order: prologue [scales q0, weights of
                // steps 0..RD-3, activations of step 0, weights of step RD-2];
                // step s, after its barrier: activations of step s+1, [scales
                // of quad q+1 if s % 4 == 0], weights of step s+RD-1.  The wait
                // at the start of step s leaves in flight the weight and scale
                // loads requested after step s's activations.
                if (u == 1) wait_vm<2 * CTW>();
                else wait_vm<CTW>();
            } else {
                // Step t requests the activations and weights of step t+3
                // (and at t % 4 == 0 the next quad's scales): at the start of
                // step s everything through step s-3's requests is complete,
                // the requests of steps s-2 and s-1 stay in flight.
                if (u == 1 || u == 2) wait_vm<2 * (DA + CTW) + CTW>();
                else wait_vm<2 * (DA + CTW)>();
            }
            lds_barrier();
            dma_a(s + NS - 1, stage(std::integral_constant<int, v + NS - 1>()));
            if (u == 0) load_sw(q + qs + 1, qs ^ 1);
            load_b(s + RD - 1, (v + RD - 1) % RD);
            const uint8_t* cur = stage(std::integral_constant<int, v>());
            constexpr int slot = v % RD;
            if (s < S) {
#pragma unroll
                for (int u4 = 0; u4 < 4; ++u4) {
                    half8 ah[RTW], bh[CTW];
#pragma unroll
                    for (int rt = 0; rt < RTW; ++rt)
                        ah[rt] = *reinterpret_cast<const half8*>(cur + (u4 * RTW + rt) * 1024 + 16 * lane);
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) {
                        const uint32_t sword = u < 2 ? sw[qs][ct][0] : sw[qs][ct][1];
                        const uint32_t sb = (sword >> (16 * (u & 1) + (u4 < 2 ? 0 : 8))) & 0xFFu;
                        bh[ct] = dequant8(word(ring[slot][ct], u4), scale_h(sb));
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                        for (int ct = 0; ct < CTW; ++ct)
                            acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bh[ct], acc[rt][ct], 0, 0, 0);
                }
            }
        };
        step(std::integral_constant<int, 0>());
        step(std::integral_constant<int, 1>());
        step(std::integral_constant<int, 2>());
        step(std::integral_constant<int, 3>());
        step(std::integral_constant<int, 4>());
        step(std::integral_constant<int, 5>());
        step(std::integral_constant<int, 6>());
        step(std::integral_constant<int, 7>());
    }
    wait_vm<0>();

    // ---- Fold: lane holds rows 16rt + 4g + r of channel 16(cw+ct) + i ----
    // f = sx v0 + sr v1 per token (compensated: rows 2m, 2m + 1 are x and r of
    // token m), sx v per row (plain); y = s_gw f
    constexpr int FV = COMP ? 2 : 4;
    float f[RTW][CTW][FV];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const int R0 = TM * rtile + 16 * rt + 4 * g + 2 * pr;
            if (COMP) {
                const int m = R0 >> 1;
                float sx = 0.0f, sr = 0.0f;
                if (m < p.M) {
                    sx = *reinterpret_cast<const float*>(p.act + (int64_t)m * p.row_bytes);
                    sr = *reinterpret_cast<const float*>(p.act + (int64_t)(p.M + m) * p.row_bytes);
                }
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) f[rt][ct][pr] = sx * acc[rt][ct][2 * pr] + sr * acc[rt][ct][2 * pr + 1];
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int m = R0 + h;
                    const float sx = m < p.M ? *reinterpret_cast<const float*>(p.act + (int64_t)m * p.row_bytes) : 0.0f;
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) f[rt][ct][2 * pr + h] = sx * acc[rt][ct][2 * pr + h];
                }
            }
        }
    }

    if (p.ks > 1) {
        // Split K: publish this slice's folded partial sums, count the slice
        // in, and let the wave that completes the count add all slices'
        // partials in slice order (the result does not depend on arrival
        // order), clear the counter for the next call, then store.  The
        // workspace is accessed with device-scope atomics only (through to the
        // memory side that all XCDs share), and the partial's stores complete
        // before the count.
        constexpr int NVAL = RTW * CTW * FV;
        const int64_t wt = tile * NW + wave;
        float* rec = p.part + (wt * p.ks + split) * (NVAL * 64) + lane;
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int j = 0; j < FV; ++j)
                    __hip_atomic_store(rec + ((rt * CTW + ct) * FV + j) * 64, f[rt][ct][j], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(p.cnt + wt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __builtin_amdgcn_readfirstlane(old);
        if (old != p.ks - 1) return;
        float tot[RTW][CTW][FV];
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int j = 0; j < FV; ++j) tot[rt][ct][j] = 0.0f;
        // the loads of QB slices' partials are in flight together (at most 64
        // values per lane; one slice at a time, each waiting for the last,
        // cost a memory round trip per slice)
        constexpr int QB = NVAL >= 64 ? 1 : 64 / NVAL;
        for (int q0 = 0; q0 < p.ks; q0 += QB) {
            float t[QB][RTW][CTW][FV];
#pragma unroll
            for (int u = 0; u < QB; ++u) {
                const int q = q0 + u < p.ks ? q0 + u : p.ks - 1;   // only q0 + u < ks is added
                const float* rq = p.part + (wt * p.ks + q) * (NVAL * 64) + lane;
#pragma unroll
                for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                        for (int j = 0; j < FV; ++j)
                            t[u][rt][ct][j] = q == split ? f[rt][ct][j]
                                                         : __hip_atomic_load(rq + ((rt * CTW + ct) * FV + j) * 64,
                                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int u = 0; u < QB; ++u)
                if (q0 + u < p.ks)
#pragma unroll
                    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
                        for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                            for (int j = 0; j < FV; ++j) tot[rt][ct][j] += t[u][rt][ct][j];
        }
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
                for (int j = 0; j < FV; ++j) f[rt][ct][j] = tot[rt][ct][j];
        if (lane == 0) __hip_atomic_store(p.cnt + wt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- store ----
    const float s_gw = reinterpret_cast<const WHeader*>(p.blob)->s_g;
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) {
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int64_t n = 16 * (cw + ct) + i;
            if (n >= p.N) continue;
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const int R0 = TM * rtile + 16 * rt + 4 * g + 2 * pr;
                if (COMP) {
                    const int m = R0 >> 1;
                    if (m < p.M) store_y(p.y, (int64_t)m * p.N + n, s_gw * f[rt][ct][pr], p.out_bf16);
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int m = R0 + h;
                        if (m < p.M) store_y(p.y, (int64_t)m * p.N + n, s_gw * f[rt][ct][2 * pr + h], p.out_bf16);
                    }
                }
            }
        }
    }
}

}  // namespace

int64_t act_tile_bytes(int fmt, int64_t B, int64_t K) {
    if (fmt == kNV) return (B + 15) / 16 * num_steps(K) * 4096;
    return (B + 15) / 16 * group_bytes(kMX, K);
}

hipError_t launch_act_tile(int fmt, bool comp, const void* act, int64_t row_bytes, int M, int64_t K, void* out,
                           hipStream_t s) {
    const int64_t B = comp ? 2 * (int64_t)M : M;
    const int64_t groups = (B + 15) / 16;
    const uint8_t* a = static_cast<const uint8_t*>(act);
    uint8_t* o = static_cast<uint8_t*>(out);
    if (fmt == kNV) {
        const dim3 grid((unsigned)((groups * num_steps(K) * 64 + 255) / 256));
        if (comp) hipLaunchKernelGGL((act_tile_f16_kernel<true>), grid, dim3(256), 0, s, a, row_bytes, M, K, groups, o);
        else hipLaunchKernelGGL((act_tile_f16_kernel<false>), grid, dim3(256), 0, s, a, row_bytes, M, K, groups, o);
    } else {
        const dim3 grid((unsigned)((groups * num_quads(K) * 320 + 255) / 256));
        if (comp) hipLaunchKernelGGL((act_tile_kernel<true>), grid, dim3(256), 0, s, a, row_bytes, M, K, groups, o);
        else hipLaunchKernelGGL((act_tile_kernel<false>), grid, dim3(256), 0, s, a, row_bytes, M, K, groups, o);
    }
    return hipGetLastError();
}

namespace {

// Waves of an NVFP4 product workgroup, 32 channels each: 8 (256 channels, one
// activation stage shared by twice the channels) from 16384 channels, else 4
// (more tiles where channels are few; measured at M = 128, K = 8192,
// N = 28672: 103 against 111 us, and at M = 128, K = N = 4096: 30.3
// against 27.0 us).
int nv_waves(int64_t N) { return num_groups(N) >= 1024 ? 8 : 4; }

// Rows of the NVFP4 product's tiles: 64 up to 64 operand rows and from 97
// to 128, and up to 256 rows where N is below 16384 (few channel tiles:
// K = N = 4096 at 256 rows 22.3 against 26.9 us, K = 14336, N = 4096 42.9
// against 47.1 us); else 128.  At 65..96 rows and wide N one 128-row tile
// reads the weights once and splits K where its tiles are few, against two
// 64-row tiles reading them twice (K = 8192, N = 28672, compensated: 60.3-61.0
// against 64.3-64.7 us at 68 rows, 58.3-58.6 against 62.9-66.0 at 80,
// 60.7-62.3 against 64.6-65.7 at 96; plain at 80 rows 63.8 against 64.2-64.7);
// from 100 rows the plain product is 4-5 % slower on one tile (67.9-72.1
// against 64.5-69.2 us at 100 and 120), and at 128 the two are within 3 %.
// At N = 28672 and 256 rows the 128-row tiles are 2-3 % faster, and at 512
// rows the two are mixed.
int nv_tile_rows(int64_t B, int64_t N) {
    return B <= 64 || (B > 96 && B <= 128) || (B <= 256 && num_groups(N) < 1024) ? 64 : 128;
}
int64_t nv_tiles(int64_t B, int64_t N) {
    const int tm = nv_tile_rows(B, N), nw = nv_waves(N);
    return (B + tm - 1) / tm * ((num_groups(N) + nw * 2 - 1) / (nw * 2));
}

// Steps per slice of a split into ks slices: a multiple of 8 (the product's
// loop body), so that ceil(S / slice) slices cover S.
int slice_steps(int64_t S, int ks) { return (int)(((S + ks - 1) / ks + 7) & ~(int64_t)7); }

}  // namespace

// Split K while the tiles x slices stay within one workgroup per compute unit
// and the slices hold at least 8 steps (measured at M = 64, K = 14336,
// N = 4096, 64 tiles: 67 us unsplit, 40 us in 2 slices, 28 us in 4).
int nv_tile_split(int64_t B, int64_t N, int64_t K, int num_cus) {
    const int64_t tiles = nv_tiles(B, N), S = num_steps(K);
    int ks = 1;
    while (ks < kMaxTileSplit && tiles * 2 * ks <= num_cus && S >= 16 * ks && tiles * nv_waves(N) <= kSplitGroups)
        ks *= 2;
    return ks <= 1 ? 1 : (int)((S + slice_steps(S, ks) - 1) / slice_steps(S, ks));
}

// Folded partial sums per tile, wave and slice: the tile's 16-row tiles x 2
// channel groups x 64 lanes x 2 values per lane (compensated: one per token of
// each pair of rows) or 4 (plain).
int64_t nv_split_bytes(int64_t B, int64_t N, int ks, bool comp) {
    return ks <= 1 ? 0 : nv_tiles(B, N) * nv_waves(N) * ks * (nv_tile_rows(B, N) / 16) * 2 * (comp ? 2 : 4) * 64 * 4;
}

hipError_t launch_gemm_tile_dma_nv(bool comp, const void* act_tiled, const void* act, int64_t row_bytes,
                                   const void* blob, int M, int64_t N, int64_t K, void* y, bool out_bf16,
                                   int ks, int* cnt, float* part, hipStream_t s) {
    NvArgs a{static_cast<const uint8_t*>(act_tiled), static_cast<const uint8_t*>(act), row_bytes,
             static_cast<const uint8_t*>(blob), M, N, K, y, out_bf16 ? 1 : 0, TileGrid{}, 1, 0, cnt, part};
    const int64_t S = num_steps(K);
    a.sl = (int)S;
    if (ks > 1) {
        a.sl = slice_steps(S, ks);
        a.ks = (int)((S + a.sl - 1) / a.sl);
    }
    const int64_t B = comp ? 2 * (int64_t)M : M;
    const int tm = nv_tile_rows(B, N);
    const int nw = nv_waves(N);
    a.grid = tile_grid(B, N, tm, 16 * 2 * nw);
    a.grid.tiles *= a.ks;
    a.grid.per_xcd = (a.grid.tiles + kXcds - 1) / kXcds;
    const dim3 grid((unsigned)(a.grid.per_xcd * kXcds));
    // 64-row tiles: four activation stages (64 KB of LDS, two workgroups per
    // CU); 128-row tiles: two (64 KB)
    auto run = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(64 * nw), 0, s, a); };
    if (tm == 64 && nw == 4) {
        if (comp) run(gemm_tile_nv_dma<true, 4, 2, 4, 4>);
        else run(gemm_tile_nv_dma<false, 4, 2, 4, 4>);
    } else if (tm == 64) {
        if (comp) run(gemm_tile_nv_dma<true, 4, 2, 4, 8>);
        else run(gemm_tile_nv_dma<false, 4, 2, 4, 8>);
    } else if (nw == 4) {
        if (comp) run(gemm_tile_nv_dma<true, 8, 2, 2, 4>);
        else run(gemm_tile_nv_dma<false, 8, 2, 2, 4>);
    } else {
        if (comp) run(gemm_tile_nv_dma<true, 8, 2, 2, 8>);
        else run(gemm_tile_nv_dma<false, 8, 2, 2, 8>);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_tile_dma(bool comp, const void* act_tiled, const void* blob, int M, int64_t N, int64_t K,
                                void* y, bool out_bf16, int num_cus, hipStream_t s) {
    DmaArgs a{static_cast<const uint8_t*>(act_tiled), static_cast<const uint8_t*>(blob), M, N, K, y,
              out_bf16 ? 1 : 0, TileGrid{}};
    return comp ? launch_mx_tiles<true>(a, num_cus, s) : launch_mx_tiles<false>(a, num_cus, s);
}

}  // namespace rsfp4
