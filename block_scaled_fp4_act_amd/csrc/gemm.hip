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
// thread-local fp32 operation (the idea of the row-pair packing of Figure 5,
// realised with MFMA lane ownership instead of TMEM loads).  The NVFP4 row
// scales s_x, s_r are constants along K, so each wave folds its partial sums,
// s_x Z_m + s_r Z_{M+m}, before they leave registers.
//
// Work decomposition (one design for all M <= 16, i.e. B <= 32; one launch
// covers up to 16 waves x 8 steps = 16384 elements of K, and longer K runs as
// two launches over consecutive step ranges, the second adding to y):
//   * a workgroup owns groups of 16 output channels (grid-stride over groups)
//     and KW waves that split K: wave w owns steps [w*MAXS, w*MAXS + MAXS) of
//     128 elements (MAXS a power of two, so a wave's steps sit inside one
//     4-step quad of the weight layout, or fill whole quads);
//   * a wave loads its activation fragments ONCE (they stay in VGPRs across
//     all groups; NVFP4 dequantizes them to f16 once where registers allow),
//     then streams the packed weights: per step one 16-byte load per lane =
//     1 KB per wave, fully coalesced, and per group one load for the block
//     scales of all its steps.  The loads of the next PD groups are in flight
//     while a group is computed (register ring);
//   * NVFP4: each 8-element run is dequantized in registers to f16 with its
//     E4M3 block scale (e * S_b has <= 6 significant bits and lies in
//     [2^-10, 2688], so f16 holds it exactly) and fed to
//     v_mfma_f32_16x16x32_f16; the fp32 tensor scales s_gx, s_gr, s_gw are
//     applied in the Fold epilogue;
//   * MXFP4: codes and E8M0 scales go straight into the native block-scaled
//     v_mfma_scale_f32_16x16x128_f8f6f4 (FP4 x FP4, one scale per lane = per
//     32-element block), no dequantization at all;
//   * the KW partial accumulators of a group meet in LDS (compensated: already
//     folded, half the bytes); the last wave to deposit its partial (an LDS
//     counter per group) sums the KW partials in a fixed order
//     (deterministic), scales and stores, so no barrier is needed while groups
//     are streamed.  When a workgroup owns more groups than LDS
//     slots, the slots are recycled after a workgroup barrier.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "codec.h"
#include "fp4_frag.h"
#include "kernels.h"
#include "layout.h"
#include "quant_row.h"

namespace rsfp4 {

namespace {

constexpr int kMaxWaves = 16;
constexpr int kRedBytesMax = 128 * 1024;   // LDS for partial sums per workgroup
constexpr int kLdsPerCu = 160 * 1024;      // gfx950
constexpr int kLdsInq = 150 * 1024;        // partials + records, quantizing in the workgroup

// Scale bytes of a wave's MAXS steps, per lane: NVFP4 2 bytes per step, MXFP4
// 1.  Up to four steps sit in one quad entry and come with one load; eight
// steps span two quads and take two.
template <int FMT, int MAXS>
struct ScaleWord {
    static constexpr int kBytesPerQuad = (MAXS < 4 ? MAXS : 4) * (FMT == kNV ? 2 : 1);
    static constexpr int kQuads = MAXS > 4 ? 2 : 1;
    static constexpr int kWordsPerQuad = kBytesPerQuad > 4 ? 2 : 1;
    uint32_t w[kQuads * kWordsPerQuad];
    // the scale byte of step t, block h (NVFP4 h = 0/1; MXFP4 h = 0)
    __device__ __forceinline__ uint32_t byte(int t, int h) const {
        const int q = t >> 2, tq = t & 3;
        const int bit = FMT == kNV ? 16 * tq + 8 * h : 8 * tq;
        return (w[q * kWordsPerQuad + (bit >> 5)] >> (bit & 31)) & 0xFFu;
    }
};

// CPOL: the loads' cache-policy bits (kStreamPolicy marks the weight stream
// non-temporal).
template <int FMT, int MAXS, int CPOL>
__device__ __forceinline__ void load_scales(__amdgpu_buffer_rsrc_t r, const uint32_t* off,
                                            ScaleWord<FMT, MAXS>& s) {
    using SW = ScaleWord<FMT, MAXS>;
#pragma unroll
    for (int q = 0; q < SW::kQuads; ++q) {
        if (SW::kBytesPerQuad == 1) {
            s.w[q] = __builtin_amdgcn_raw_buffer_load_b8(r, off[q], 0, CPOL);
        } else if (SW::kBytesPerQuad == 2) {
            s.w[q] = __builtin_amdgcn_raw_buffer_load_b16(r, off[q], 0, CPOL);
        } else if (SW::kBytesPerQuad == 4) {
            s.w[q] = __builtin_amdgcn_raw_buffer_load_b32(r, off[q], 0, CPOL);
        } else {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off[q], 0, CPOL);
            s.w[2 * q] = v[0];
            s.w[2 * q + 1] = v[1];
        }
    }
}

struct GemmArgs {
    const uint8_t* act;
    int64_t row_bytes;
    const uint8_t* blob;
    int M;
    int64_t N;
    int64_t K;
    void* y;          // fp32 or (out_bf16) bf16 output
    int ngl;          // LDS slots for partial sums (groups in flight per workgroup)
    int s_lo;         // first K step of this launch (wave w owns s_lo + w*MAXS ..)
    int64_t k_hi;     // K elements at or past k_hi are left to another launch
    int accum;        // add to y instead of overwriting it (fp32 output only)
    int out_bf16;     // store y as bf16 (round to nearest even)
    const void* x;    // in-workgroup quantization: the input rows x[M, K]
    int qrow;         // threads per quantized row (a multiple of 64)
    // grouped (mixture of experts), offsets non-null: blockIdx.y is the expert
    // e, its rows offsets[e] .. offsets[e+1] of the act buffer (of M_total rows;
    // at most M of them are computed) and its blob the e-th of the stacked
    // blobs, blob_stride bytes apart
    const int32_t* offsets;
    int64_t blob_stride;
    int M_total;
    int E;
    // split K (ks > 1): workgroup b owns slice b % ks, steps s_lo + (b % ks) * ss
    // .. + ss, and the groups b / ks + j * (grid / ks); the slices' partial sums
    // meet in ws (counters cnt[G], then one record per group and slice)
    int ks;
    int ss;
    int* cnt;
    float* ws;
};

// APRE: the activation fragments are dequantized to f16 once, before the
// weight stream starts (NVFP4 only; 16 VGPRs per step and row tile), so the
// streaming loop only dequantizes weights.  Without it they stay as codes and
// are dequantized at each use.
// PD: weight prefetch depth.  The loads of group j + PD are issued before group
// j is computed, through a ring of PD + 1 register buffers (the loop is
// unrolled by PD + 1 so every buffer index is static).
// RM: how the KW partial sums of a group are combined.  RM = 0: the last wave
// to deposit its partial (LDS counter) reduces the group at once.  RM = 1: the
// partials of up to ngl groups wait in LDS and the waves reduce them together
// after one barrier (one group per wave).
//
// ST (streaming order, for plans whose workgroups stream many weight bytes):
// the weight loads are non-temporal (each byte is read once, so it should not
// displace the activation records from the caches), a group's block scales
// are loaded before its codes (the first step's dequantization needs them,
// and the memory counter returns loads in order, so the MFMAs of step t can
// start as soon as steps 0..t have arrived instead of after the whole group),
// the first weight loads of a prefetching plan are issued before the
// activation loads (a single pass, PD = 0, loads the activation fragments
// first: the in-order memory counter would otherwise hold every step's
// arithmetic until the last weight byte), and the next group's loads are
// pinned ahead of the current group's arithmetic.  Measured
// at K = 8192, N = 28672 (M = 8): 5-8 % from the cache policy, a further
// 4-5 % from the ordering.  Single-group plans with few steps per wave keep
// the plain order (their loads are all issued at once anyway).
//
// XT (void: the activation records come from act in global memory): every
// workgroup quantizes the M input rows x[M, K] (dtype XT) itself, with the
// quantizer's row routine, into records in its LDS -- the same bytes the
// quantize kernel writes -- and reads its fragments from there.  The rows are
// quantized in parallel, p.qrow threads per row, NCQ chunks of 8 per thread;
// the x loads go out before the weight loads (the memory counter is in order)
// and the quantization runs while the weights are in flight.  Every workgroup
// repeats the same quantization, on a compute unit that would otherwise wait
// for its weights; no workgroup depends on another.
// XS: K split across workgroups (p.ks > 1; the partial sums meet in p.ws).
template <int FMT, int MAXS, int RT, bool COMP, int PD, bool APRE, int RM, bool ST, bool XS = false,
          typename XT = void, int NCQ = 1>
__global__ __launch_bounds__(1024) void gemm_small_kernel(GemmArgs p) {
    constexpr bool kInq = !std::is_void<XT>::value;
    using XIn = std::conditional_t<kInq, XT, float>;
    // LDS: [ngl] counters (padded to 64), then [ngl][KW][RT][4][64] partial sums
    extern __shared__ float lds[];
    constexpr bool kPre = APRE && FMT == kNV;
    constexpr int kAC = kPre ? 1 : MAXS;     // code registers kept per row tile
    constexpr int kAH = kPre ? MAXS : 1;     // f16 fragments kept per row tile
    constexpr int NB = PD + 1;               // weight buffers in the ring
    constexpr int PW = COMP ? 2 : 4;         // partial sums per lane and row tile in LDS
    using SW = ScaleWord<FMT, MAXS>;
    constexpr int64_t SB1 = scale_bytes_per_step_lane(FMT);

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int KW = blockDim.x >> 6;
    const int g = lane >> 4, i = lane & 15;
    const int ks = XS ? (int)(blockIdx.x % (unsigned)p.ks) : 0;    // K slice of this workgroup
    const int s_base = XS ? p.s_lo + ks * p.ss : p.s_lo;
    const int s0 = s_base + wave * MAXS;          // this wave's first step
    // K elements at or past k_hi belong to another slice or launch
    const int64_t k_hi = XS && (int64_t)(s_base + p.ss) * kStepK < p.k_hi ? (int64_t)(s_base + p.ss) * kStepK : p.k_hi;
    const int64_t G = num_groups(p.N);
    const int64_t GB = group_bytes(FMT, p.K);
    const uint32_t scale_base = (uint32_t)(kActHead + p.K / 2);
    const int64_t grid = XS ? gridDim.x / p.ks : gridDim.x;       // the group stride
    const int64_t c0 = XS ? blockIdx.x / p.ks : blockIdx.x;
    const int ngl = p.ngl;
    int* counters = reinterpret_cast<int*>(lds);
    float* red = lds + ((ngl + 63) & ~63);
    // in-workgroup quantization: the B activation records after the partials
    uint8_t* act_lds = reinterpret_cast<uint8_t*>(red + ngl * KW * RT * PW * 64);

    // this workgroup's rows: mb .. mb + Mr - 1 of an act buffer of Mt rows
    int mb = 0, Mr = p.M, Mt = p.M;
    const uint8_t* blob = p.blob;
    if (p.offsets) {
        const int e = blockIdx.y;
        Mt = p.M_total;
        const int lo = min(max(p.offsets[e], 0), Mt);
        const int hi = min(max(p.offsets[e + 1], lo), Mt);
        mb = lo;
        Mr = min(hi - lo, p.M);
        blob += (int64_t)e * p.blob_stride;
    }

    float s_gw = 1.0f;
    if (FMT == kNV) s_gw = reinterpret_cast<const WHeader*>(blob)->s_g;

    // Offsets of this wave's loads inside a group: steps past the padded end
    // of the group land past its last byte, i.e. out of range (zeros).
    const uint32_t code_base = (uint32_t)step_code_offset(FMT, s0) + 16u * lane;
    uint32_t sc_off[SW::kQuads];
#pragma unroll
    for (int q = 0; q < SW::kQuads; ++q)
        sc_off[q] = (uint32_t)(quad_scale_offset(FMT, s0 + 4 * q) + lane * 4 * SB1 + (s0 % 4) * SB1);

    uint4 wb[NB][MAXS];
    SW wsc[NB];

    // One buffer resource per group (32-bit lane offsets, no 4 GB limit
    // overall).  Every load is issued unconditionally: a step past the end, or a
    // group past the end (zero-sized resource), reads out of range and the
    // buffer unit returns zeros.  Without branches around the loads the
    // compiler's memory-counter waits stay exact, so prefetched groups are
    // really in flight while earlier ones are computed.
    constexpr int WPOL = ST ? kStreamPolicy : 0;
    auto load_w = [&](int64_t c, uint4 (&codes)[MAXS], SW& sc) {
        const bool live = c < G;
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(blob + kWHeader + (live ? c : 0) * GB), (short)0, live ? (int)GB : 0, kRsrcWord3);
        if (ST) load_scales<FMT, MAXS, WPOL>(r, sc_off, sc);
#pragma unroll
        for (int t = 0; t < MAXS; ++t)
            codes[t] = ld128<WPOL>(r, code_base + (uint32_t)((t / 4) * quad_bytes(FMT) + (t % 4) * kStepCodes));
        if (!ST) load_scales<FMT, MAXS, WPOL>(r, sc_off, sc);
    };

    // in-workgroup quantization: this thread's row and chunks of x, loaded
    // before any weight load
    const int qrow = kInq ? p.qrow : 64;
    const int mq = kInq ? (int)threadIdx.x / qrow : 0;
    const bool qactive = kInq && mq < p.M;
    const int qlt = qactive ? (int)threadIdx.x % qrow : lane;
    const int qnt = qactive ? qrow : 64;
    float xq[NCQ][8];
    if constexpr (kInq)
        row_load<NCQ, 8, XIn>(static_cast<const XIn*>(p.x) + (int64_t)(qactive ? mq : 0) * p.K, p.K, qlt, qnt, qactive, xq);
    auto quantize_rows = [&](float (*qred)[kQMaxThreads / 64]) {
        row_quantize<FMT, NCQ, 8>(xq, p.K, qlt, qnt, qactive, COMP ? 1 : 0, act_lds + (int64_t)mq * p.row_bytes,
                                  act_lds + (int64_t)(p.M + mq) * p.row_bytes, qred);
    };

    // ---- activation fragments: loaded once, kept in registers ----
    // Their loads go out first; the first groups' weight loads follow at once,
    // so both latencies overlap and the fragments can be dequantized while the
    // weights are still in flight.
    const int B = COMP ? 2 * Mt : Mt;
    const uint32_t act_bytes = (uint32_t)(B * p.row_bytes);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)p.act, (short)0, (int)act_bytes, kRsrcWord3);
    uint4 a_raw[RT][MAXS];
    uint32_t a_rsc[RT][MAXS];
    float row_s0[2 * RT], row_s1[2 * RT];
    auto load_act = [&]() {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int ti = 16 * rt + i;               // tile row of this lane's A operand
            int arow;
            bool rvalid;
            if (COMP) {
                const int m = ti >> 1;
                rvalid = m < Mr;
                arow = (ti & 1) ? Mt + mb + m : mb + m;
            } else {
                rvalid = ti < Mr;
                arow = mb + ti;
            }
#pragma unroll
            for (int t = 0; t < MAXS; ++t) {
                const int64_t k0 = kStepK * (s0 + t) + 32 * g;
                const bool in = rvalid && k0 < k_hi;     // else: out of range -> zeros
                const uint32_t rec = in ? (uint32_t)(arow * p.row_bytes) : act_bytes;
                if (kInq) {
                    const uint8_t* r8 = act_lds + rec;
                    a_raw[rt][t] = in ? *reinterpret_cast<const uint4*>(r8 + kActHead + k0 / 2) : make_uint4(0, 0, 0, 0);
                    if (FMT == kNV)
                        a_rsc[rt][t] = in ? *reinterpret_cast<const uint16_t*>(r8 + scale_base + k0 / 16) : 0u;
                    else
                        a_rsc[rt][t] = in ? r8[scale_base + k0 / 32] : 0u;
                    continue;
                }
                a_raw[rt][t] = ld128(ra, in ? rec + (uint32_t)(kActHead + k0 / 2) : act_bytes);
                if (FMT == kNV)
                    a_rsc[rt][t] = __builtin_amdgcn_raw_buffer_load_b16(ra, in ? rec + scale_base + (uint32_t)(k0 / 16) : act_bytes, 0, 0);
                else
                    a_rsc[rt][t] = __builtin_amdgcn_raw_buffer_load_b8(ra, in ? rec + scale_base + (uint32_t)(k0 / 32) : act_bytes, 0, 0);
            }
        }

        // NVFP4 tensor scales of the rows this lane folds and stores (the
        // epilogue's only global reads), fetched with the fragments: item (rt, pr)
        // covers tile rows ti0 = 16rt + 4g + 2pr and ti0 + 1, i.e. token row ti0/2
        // (base and residue) when compensated, rows ti0 and ti0 + 1 otherwise.
#pragma unroll
        for (int item = 0; item < 2 * RT; ++item) {
            row_s0[item] = row_s1[item] = 0.0f;
            if (FMT == kNV) {
                const int ti0 = 16 * (item >> 1) + 4 * g + 2 * (item & 1);
                const int r0 = mb + (COMP ? ti0 >> 1 : ti0);
                const int r1 = COMP ? Mt + mb + (ti0 >> 1) : mb + ti0 + 1;
                const bool v0 = COMP ? (ti0 >> 1) < Mr : ti0 < Mr;
                const bool v1 = COMP ? v0 : ti0 + 1 < Mr;
                if (kInq) {
                    row_s0[item] = v0 ? *reinterpret_cast<const float*>(act_lds + r0 * p.row_bytes) : 0.0f;
                    row_s1[item] = v1 ? *reinterpret_cast<const float*>(act_lds + r1 * p.row_bytes) : 0.0f;
                    continue;
                }
                row_s0[item] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    ra, v0 ? (uint32_t)(r0 * p.row_bytes) : act_bytes, 0, 0));
                row_s1[item] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                    ra, v1 ? (uint32_t)(r1 * p.row_bytes) : act_bytes, 0, 0));
            }
        }
    };
    // The first group's weights are requested in the prologue at any prefetch
    // depth (with PD = 0 the loop then skips its load of group 0), so no
    // workgroup waits for its activation fragments before its weight stream
    // starts.
    constexpr int PRE = PD > 0 ? PD : 1;
    if (ST && PD > 0 && !kInq) {
#pragma unroll
        for (int q = 0; q < PRE; ++q) load_w(c0 + q * grid, wb[q], wsc[q]);
        load_act();
    } else {
        if (!kInq) load_act();
#pragma unroll
        for (int q = 0; q < PRE; ++q) load_w(c0 + q * grid, wb[q], wsc[q]);
    }

    // the deferred reduction (RM = 1) uses no counters
    if (RM == 0)
        for (int k = threadIdx.x; k < ngl; k += blockDim.x) counters[k] = 0;

    if constexpr (kInq) {
        // row mq of x by threads lt = 0 .. qrow - 1 of its group; threads past
        // the M groups form one-wave groups of no row (they only take part in
        // the barriers).  The x loads were issued first (above the weights).
        __shared__ float qred[2][kQMaxThreads / 64];
        quantize_rows(qred);
        __syncthreads();                           // the records are complete
        load_act();
    }

    uint4 a_codes[RT][kAC];
    uint32_t a_sc[RT][kAC];
    half8 a_h[RT][kAH][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (kPre) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    a_h[rt][t][u] = dequant8(word(a_raw[rt][t], u), scale_h((a_rsc[rt][t] >> (u < 2 ? 0 : 8)) & 0xFFu));
            } else {
                a_codes[rt][t] = a_raw[rt][t];
                a_sc[rt][t] = a_rsc[rt][t];
            }
        }
    }
    if (RM == 0) __syncthreads();                 // counters are zero

    // ---- fold and store the group reduced from LDS slot `slot` (one wave) ----
    // The workgroup's sum of its waves' partials (fixed wave order), PV values
    // per lane: compensated, token row (16 rt + 4 g + 2 pr) / 2 of channel i
    // per (row tile, pair); plain, tile rows ti0 and ti0 + 1.
    constexpr int PV = COMP ? 2 * RT : 4 * RT;
    // The LDS reads of the partials go out in batches of RB waves (at most 16
    // values per lane), one wait per batch, and are added in wave order.  Read
    // one at a time, each waiting for the previous one, they cost 5-10 % of
    // the linear at K = 4096 and 14336 with eight or fourteen waves (MLP down,
    // M = 8: 12.35 against 11.16 us) and 1-2 % at K = 8192.
    constexpr int RB = PV >= 16 ? 1 : 16 / PV;
    auto reduce_slot = [&](int64_t c, int slot) {
        // value k of wave w's partial at base[(w * PV + k) * 64]
        const float* base = red + slot * KW * PV * 64 + lane;
        float pv[PV];
#pragma unroll
        for (int k = 0; k < PV; ++k) pv[k] = 0.0f;
        for (int w0 = 0; w0 < KW; w0 += RB) {
            float t[RB][PV];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                const int w = w0 + u < KW ? w0 + u : KW - 1;   // in range; only w0 + u < KW is added
#pragma unroll
                for (int k = 0; k < PV; ++k) t[u][k] = base[(w * PV + k) * 64];
            }
#pragma unroll
            for (int u = 0; u < RB; ++u)
                if (w0 + u < KW)
#pragma unroll
                    for (int k = 0; k < PV; ++k) pv[k] += t[u][k];
        }
        if constexpr (XS) {
            // Split K: publish this slice's partial, count it in, and let the
            // slice that completes the count sum all slices' partials in slice
            // order (so the result does not depend on arrival order), clear the
            // counter for the next call and store y.  Every access to the
            // workspace is a device-scope atomic: the partials are stored and
            // loaded with device-scope coherence (written through to, and read
            // from, the memory side shared by all XCDs instead of one XCD's
            // L2), and the wave waits for its partial stores to complete before
            // its counter increment, so a slice that sees the count complete
            // reads every other slice's finished partial.  A release/acquire
            // fence pair would also write back and invalidate this XCD's whole
            // L2 at every handoff, which measured 4-5 us per handoff.
            float* rec = p.ws + ((c * p.ks + ks) * PV) * 64 + lane;
#pragma unroll
            for (int k = 0; k < PV; ++k) __hip_atomic_store(rec + k * 64, pv[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            int old = 0;
            if (lane == 0) old = __hip_atomic_fetch_add(p.cnt + c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            old = __builtin_amdgcn_readfirstlane(old);
            if (old != p.ks - 1) return;
            // the loads of up to QB slices' partials are in flight together (at
            // most 8 values per lane)
            constexpr int QB = PV >= 8 ? 1 : 8 / PV;
            float tot[PV];
#pragma unroll
            for (int k = 0; k < PV; ++k) tot[k] = 0.0f;
            for (int q0 = 0; q0 < p.ks; q0 += QB) {
                float t[QB][PV];
#pragma unroll
                for (int u = 0; u < QB; ++u) {
                    const int q = q0 + u < p.ks ? q0 + u : p.ks - 1;   // only q0 + u < ks is added
                    const float* rq = p.ws + ((c * p.ks + q) * PV) * 64 + lane;
#pragma unroll
                    for (int k = 0; k < PV; ++k)
                        t[u][k] = q == ks ? pv[k] : __hip_atomic_load(rq + k * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
#pragma unroll
                for (int u = 0; u < QB; ++u)
                    if (q0 + u < p.ks)
#pragma unroll
                        for (int k = 0; k < PV; ++k) tot[k] += t[u][k];
            }
#pragma unroll
            for (int k = 0; k < PV; ++k) pv[k] = tot[k];
            if (lane == 0) __hip_atomic_store(p.cnt + c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int item = 0; item < 2 * RT; ++item) {
            const int rt = item >> 1, pr = item & 1;
            const int ti0 = 16 * rt + 4 * g + 2 * pr;    // tile rows ti0, ti0 + 1
            const int64_t n = c * kGroupN + i;
            if (COMP) {
                const int m = ti0 >> 1;
                if (n < p.N && m < Mr) {
                    float out = FMT == kNV ? s_gw * pv[item] : pv[item];
                    const int64_t yi = (int64_t)(mb + m) * p.N + n;
                    if (p.accum) out += reinterpret_cast<const float*>(p.y)[yi];
                    store_y(p.y, yi, out, p.out_bf16);
                }
                continue;
            }
            if (n < p.N) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int m = ti0 + h;
                    if (m < Mr) {
                        const float v = pv[2 * item + h];
                        float out = v;
                        if (FMT == kNV) out = s_gw * ((h ? row_s1[item] : row_s0[item]) * v);
                        const int64_t yi = (int64_t)(mb + m) * p.N + n;
                        if (p.accum) out += reinterpret_cast<const float*>(p.y)[yi];
                        store_y(p.y, yi, out, p.out_bf16);
                    }
                }
            }
        }
    };

    // ---- one group: MFMAs over this wave's steps, partial to LDS, and the
    // last wave to arrive reduces the group ----
    auto compute = [&](int64_t c, int slot, const uint4 (&w_codes)[MAXS], const SW& w_sc) {
        floatx4 acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
        for (int t = 0; t < MAXS; ++t) {
            if (FMT == kNV) {
                const _Float16 sw0 = scale_h(w_sc.byte(t, 0)), sw1 = scale_h(w_sc.byte(t, 1));
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const half8 b = dequant8(word(w_codes[t], u), u < 2 ? sw0 : sw1);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        half8 a;
                        if (kPre) {
                            a = a_h[rt][t][u];
                        } else {
                            // the empty asm keeps the compiler from hoisting this
                            // loop-invariant dequantization out of the group loop,
                            // which would hold every f16 fragment in registers
                            uint32_t ac = word(a_codes[rt][t], u), as = a_sc[rt][t];
                            asm volatile("" : "+v"(ac), "+v"(as));
                            a = dequant8(ac, scale_h((as >> (u < 2 ? 0 : 8)) & 0xFFu));
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
                        a, b, acc[rt], 4, 4, 0, (int)a_sc[rt][t], 0, (int)w_sc.byte(t, 0));
                }
            }
        }
        float* dst = red + ((slot * KW + wave) * RT) * (PW * 64);
        if (COMP) {
            // the Fold per wave: the row scales are constant along K, so
            // s_x m * Z_m + s_r m * Z_M+m folds each partial before the sum
            // over the waves (half the LDS of the unfolded pairs)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int item = 2 * rt + pr;
                    const float f = FMT == kNV ? row_s0[item] * acc[rt][2 * pr] + row_s1[item] * acc[rt][2 * pr + 1]
                                               : acc[rt][2 * pr] + acc[rt][2 * pr + 1];
                    dst[item * 64 + lane] = f;
                }
        } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(rt * 4 + r) * 64 + lane] = acc[rt][r];
        }
        if (RM == 0) {
            // publish this wave's partial, then count it in
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            int old = 0;
            if (lane == 0) old = atomicAdd(&counters[slot], 1);
            old = __builtin_amdgcn_readfirstlane(old);
            if (old == KW - 1) {                  // the last partial of this group
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                reduce_slot(c, slot);
            }
        }
    };

    // groups of this workgroup: c0, c0 + grid, ...; the loop runs a whole number
    // of ring turns and skips the work (never the loads) past the end.  Group j
    // uses LDS slot j % ngl; before the slots wrap (RM = 0), or when they are
    // full or the groups end (RM = 1), a barrier separates the partial sums of
    // the groups so far from the reuse of their slots.
    const int64_t nj = c0 < G ? (G - c0 + grid - 1) / grid : 0;
    int slot = 0;
    auto flush = [&](int64_t jlast, int nslots) {   // RM = 1
        __syncthreads();
        for (int sl = wave; sl < nslots; sl += KW) reduce_slot(c0 + (jlast - nslots + 1 + sl) * grid, sl);
        __syncthreads();
    };
    for (int64_t j0 = 0; j0 < nj; j0 += NB) {
#pragma unroll
        for (int q = 0; q < NB; ++q) {
            const int64_t j = j0 + q;
            if (PD > 0 || j > 0) load_w(c0 + (j + PD) * grid, wb[(q + PD) % NB], wsc[(q + PD) % NB]);
            // keep the compiler from sinking these loads below the arithmetic
            if (ST) __builtin_amdgcn_sched_barrier(0);
            if (j < nj) {
                if (RM == 0 && slot == ngl) {     // wrap: every slot reduced -> reset
                    __syncthreads();
                    for (int k = threadIdx.x; k < ngl; k += blockDim.x) counters[k] = 0;
                    __syncthreads();
                    slot = 0;
                }
                compute(c0 + j * grid, slot, wb[q], wsc[q]);
                ++slot;
                if (RM == 1 && (slot == ngl || j == nj - 1)) {
                    flush(j, slot);
                    slot = 0;
                }
            }
        }
    }
}

template <int FMT, int MAXS, int RT, bool COMP, int PD, bool APRE, int RM, bool ST, bool XS = false,
          typename XT = void, int NCQ = 1>
hipError_t launch_t(const GemmArgs& a, int KW, int64_t grid, hipStream_t s) {
    constexpr bool kInq = !std::is_void<XT>::value;
    // allow the LDS of a CU for the partial-sum slots and, quantizing in the
    // workgroup, the activation records (set once per kernel)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_small_kernel<FMT, MAXS, RT, COMP, PD, APRE, RM, ST, XS, XT, NCQ>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kInq ? kLdsInq : kRedBytesMax + 1024);
    if (attr != hipSuccess) return attr;
    size_t lds = (size_t)((a.ngl + 63) & ~63) * 4 + (size_t)a.ngl * KW * RT * (COMP ? 512 : 1024);
    if (kInq) lds += (size_t)(COMP ? 2 * a.M : a.M) * a.row_bytes;
    hipLaunchKernelGGL((gemm_small_kernel<FMT, MAXS, RT, COMP, PD, APRE, RM, ST, XS, XT, NCQ>),
                       dim3((unsigned)grid, a.offsets ? (unsigned)a.E : 1u), dim3(64 * KW), lds, s, a);
    return hipGetLastError();
}

// Variant table, from sweeps of prefetch depth, pre-dequantized activations,
// reduction mode and load order on the decode workloads (and the compiler's
// register counts: 128 VGPRs at 16 waves per CU).  Deep prefetch does not pay
// (depth 2 spills): one group ahead is best for NVFP4 when a workgroup streams
// several groups; MXFP4 (one MFMA per step, no dequantization) and
// single-group plans issue each group's loads just before it.  A workgroup
// with a single group and few steps per wave reduces it as soon as its last
// partial lands (RM = 0); otherwise the deferred reduction (RM = 1) is faster.
// The streaming order (ST) pays wherever a wave streams several groups or
// eight steps; single-group plans of one to four steps per wave keep the
// plain order (K = N = 4096: 5.3 against 5.6-6.0 us).
constexpr int pd_for(int fmt, int rt, int maxs, bool single) {
    if (single) return 0;
    if (fmt == kNV) return maxs <= 4 ? 1 : 0;
    return rt == 1 ? 0 : (maxs <= 2 ? 1 : 0);
}
constexpr bool apre_for(int fmt, int rt, int maxs, bool single, bool comp) {
    // one row tile: up to 4 steps per wave (compensated, or one pass over the
    // groups; 128 VGPRs at 4 steps, no spills; 6-9 % faster at K = 8192,
    // N = 28672 than dequantizing per group), 8 spill; two row tiles: 2 steps
    // fit (the compensated kernels; the plain ones spill), four never do
    return fmt == kNV && (rt == 1 ? maxs <= (single || comp ? 4 : 2) : (rt == 2 && comp && maxs <= 2));
}
constexpr bool st_for(int maxs, bool single) { return !single || maxs == 8; }
constexpr int rm_for(int maxs, bool single) { return single && !st_for(maxs, single) ? 0 : 1; }

template <int FMT, int RT, bool COMP, int MAXS>
hipError_t launch_v(const GemmArgs& a, int KW, int64_t grid, hipStream_t s, bool single) {
    // split K: compensated NVFP4 with one or two row tiles and one or two steps
    // per wave (the plans plan_gemm_small makes), streaming order, deferred
    // reduction
    if constexpr (FMT == kNV && RT <= 2 && COMP && MAXS <= 2) {
        if (a.ks > 1)
            return launch_t<FMT, MAXS, RT, COMP, pd_for(FMT, RT, MAXS, false), apre_for(FMT, RT, MAXS, false, COMP),
                            1, true, true>(a, KW, grid, s);
    }
    if (a.ks > 1) return hipErrorInvalidValue;
    if (single)
        return launch_t<FMT, MAXS, RT, COMP, pd_for(FMT, RT, MAXS, true), apre_for(FMT, RT, MAXS, true, COMP),
                        rm_for(MAXS, true), st_for(MAXS, true)>(a, KW, grid, s);
    return launch_t<FMT, MAXS, RT, COMP, pd_for(FMT, RT, MAXS, false), apre_for(FMT, RT, MAXS, false, COMP),
                    rm_for(MAXS, false), st_for(MAXS, false)>(a, KW, grid, s);
}

template <int FMT, int RT, bool COMP>
hipError_t launch_maxs(const GemmArgs& a, int maxs, int KW, int64_t grid, hipStream_t s, bool single) {
    switch (maxs) {
        case 1: return launch_v<FMT, RT, COMP, 1>(a, KW, grid, s, single);
        case 2: return launch_v<FMT, RT, COMP, 2>(a, KW, grid, s, single);
        case 4: return launch_v<FMT, RT, COMP, 4>(a, KW, grid, s, single);
        default: return launch_v<FMT, RT, COMP, 8>(a, KW, grid, s, single);
    }
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& a, int rt, bool comp, int maxs, int KW, int64_t grid,
                      hipStream_t s, bool single) {
    if (rt == 1)
        return comp ? launch_maxs<FMT, 1, true>(a, maxs, KW, grid, s, single)
                    : launch_maxs<FMT, 1, false>(a, maxs, KW, grid, s, single);
    if (rt == 2)
        return comp ? launch_maxs<FMT, 2, true>(a, maxs, KW, grid, s, single)
                    : launch_maxs<FMT, 2, false>(a, maxs, KW, grid, s, single);
    // four row tiles: compensated NVFP4 only (the host's dispatch)
    if (FMT != kNV || !comp) return hipErrorInvalidValue;
    return launch_maxs<kNV, 4, true>(a, maxs, KW, grid, s, single);
}

}  // namespace

GemmPlan plan_gemm_small(int64_t M, int64_t N, int64_t S, bool comp, int num_cus, bool split_ok) {
    GemmPlan pl;
    const int64_t B = comp ? 2 * M : M;
    pl.rt = B <= 16 ? 1 : (B <= 32 ? 2 : 4);
    const int64_t G = num_groups(N);
    // the fewest steps per wave (a power of two) that covers K with <= 16 waves;
    // compensated with one row tile and at least as many groups as compute
    // units, K of 17..32 steps takes four steps per wave over eight waves, one
    // workgroup per CU (K = 4096, N = 14336, M = 8: 9.8 against 10.4 us for
    // two steps over 16 waves; K = N = 4096, M = 4: 5.8 against 6.05 us)
    pl.maxs = S <= 16 ? 1 : (S <= 32 ? 2 : (S <= 64 ? 4 : 8));
    const bool wide4 = comp && pl.rt == 1 && S > 16 && S <= 32 && G >= num_cus;
    if (wide4) pl.maxs = 4;
    pl.kw = (int)((S + pl.maxs - 1) / pl.maxs);
    const int per_cu = wide4 ? 1 : (kMaxWaves / pl.kw > 0 ? kMaxWaves / pl.kw : 1);
    const int64_t cap = (int64_t)num_cus * per_cu;
    pl.grid = G < cap ? G : cap;
    const int64_t per_wg = (G + pl.grid - 1) / pl.grid;         // groups per workgroup
    // LDS per workgroup: at most 128 KB, and small enough for per_cu of them
    const int64_t lds_cap = kRedBytesMax < kLdsPerCu / per_cu - 1024 ? kRedBytesMax : kLdsPerCu / per_cu - 1024;
    const int64_t fit = lds_cap / ((int64_t)pl.kw * pl.rt * (comp ? 512 : 1024));
    pl.ngl = (int)(per_wg < fit ? per_wg : fit);
    if (pl.ngl < 1) pl.ngl = 1;
    if (!split_ok || pl.rt > 2 || !comp) return pl;

    // Split K across workgroups (one workgroup per CU, each owning one K slice
    // of several channel groups) where the shape makes it pay: few groups with
    // long K (G <= CUs, S >= 64): four slices, so a workgroup streams four
    // groups' slices instead of one group's whole K and holds a quarter of
    // the activation operand (K = 14336, N = 4096, M = 8: 11.8 against
    // 14.2 us).  A half round of groups (G a multiple of CUs / 2 but not of
    // CUs) split in two, which once paid, is now slower than the unsplit
    // four-steps-per-wave plan (K = 4096, N = 14336: 10.3 against 9.8 us at
    // M = 8, 10.3 against 8.7 us at M = 2).  The MXFP4 shapes and
    // K = N = 4096 are slower split (one handoff costs about as much as a
    // whole K = 4096 group).
    int ks = 0;
    if (G > kSplitGroups) return pl;
    if (pl.rt == 2) {
        // two row tiles hold their f16 fragments for two steps per wave, 32
        // steps per workgroup: slices of up to 32 steps, one pass over K
        // instead of launches of 32 steps that each read and rewrite y
        // (2 to 4 equal slices, each of at most 32 steps)
        if (S <= 32) return pl;
        for (int k = (int)((S + 31) / 32); k <= 4 && ks == 0; ++k)
            if (S % k == 0 && ((S / k) % 2 == 0 || S / k <= kMaxWaves)) ks = k;
    } else if (G <= num_cus && S >= 64 && S % 4 == 0) {
        ks = 4;
    }
    if (ks == 0) return pl;
    const int64_t ss = S / ks;
    // two steps per wave where they fit in 16 waves (MLP down: 14 waves, up:
    // 8), else one (four steps per wave spill with the split's reduction)
    int maxs = 0;
    for (int m : {2, 1})
        if (maxs == 0 && ss % m == 0 && ss / m <= kMaxWaves) maxs = m;
    if (maxs == 0) return pl;
    GemmPlan sp;
    sp.rt = pl.rt;
    sp.maxs = maxs;
    sp.kw = (int)(ss / maxs);
    sp.ks = ks;
    sp.ss = (int)ss;
    const int64_t per_slice = G * ks >= num_cus ? num_cus / ks : G;   // workgroups per slice
    sp.grid = per_slice * ks;
    const int64_t units = (G + per_slice - 1) / per_slice;           // groups per workgroup
    const int64_t sfit = kRedBytesMax / ((int64_t)sp.kw * sp.rt * 512);
    sp.ngl = (int)(units < sfit ? units : sfit);
    if (sp.ngl < 1) sp.ngl = 1;
    return sp;
}

// In-workgroup quantization (bf16 x, one row tile, up to 4 steps per wave):
// the weight prefetch and reduction as for the narrow plans, plus NCQ.
template <int FMT, bool COMP, int MAXS, int NCQ>
hipError_t launch_inq_v(const GemmArgs& a, int KW, int64_t grid, hipStream_t s, bool single) {
    using XT = __hip_bfloat16;
    if (single)
        return launch_t<FMT, MAXS, 1, COMP, 1, apre_for(FMT, 1, MAXS, true, COMP), rm_for(MAXS, true),
                        st_for(MAXS, true), false, XT, NCQ>(a, KW, grid, s);
    return launch_t<FMT, MAXS, 1, COMP, 1, apre_for(FMT, 1, MAXS, false, COMP), rm_for(MAXS, false),
                    st_for(MAXS, false), false, XT, NCQ>(a, KW, grid, s);
}

template <int FMT, bool COMP>
hipError_t launch_inq_fmt(const GemmArgs& a, int maxs, int ncq, int KW, int64_t grid, hipStream_t s, bool single) {
    if (ncq <= 2) {
        switch (maxs) {
            case 1: return launch_inq_v<FMT, COMP, 1, 2>(a, KW, grid, s, single);
            case 2: return launch_inq_v<FMT, COMP, 2, 2>(a, KW, grid, s, single);
            default: return launch_inq_v<FMT, COMP, 4, 2>(a, KW, grid, s, single);
        }
    }
    switch (maxs) {
        case 1: return launch_inq_v<FMT, COMP, 1, 4>(a, KW, grid, s, single);
        case 2: return launch_inq_v<FMT, COMP, 2, 4>(a, KW, grid, s, single);
        default: return launch_inq_v<FMT, COMP, 4, 4>(a, KW, grid, s, single);
    }
}

int64_t split_ws_bytes(const GemmPlan& pl, bool comp, int64_t N) {
    if (pl.ks <= 1) return 0;
    const int64_t G = num_groups(N);
    const int64_t pv = comp ? 2 * pl.rt : 4 * pl.rt;           // partial sums per lane
    return kSplitCounterBytes + G * pl.ks * pv * 64 * 4;
}

hipError_t launch_gemm_small(int fmt, const GemmPlan& pl, bool comp, const void* act,
                             int64_t row_bytes, const void* blob, int M, int64_t N, int64_t K,
                             void* y, bool out_bf16, int s_lo, int s_hi, bool accum, void* ws, hipStream_t s) {
    const int64_t k_hi = (int64_t)s_hi * kStepK < K ? (int64_t)s_hi * kStepK : K;
    if (pl.ks > 1 && (ws == nullptr || pl.grid % pl.ks != 0 || pl.ss * pl.ks < s_hi - s_lo)) return hipErrorInvalidValue;
    int* cnt = static_cast<int*>(ws);
    if (pl.ks > 1 && num_groups(N) > kSplitGroups) return hipErrorInvalidValue;
    float* part = pl.ks > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kSplitCounterBytes) : nullptr;
    GemmArgs a{static_cast<const uint8_t*>(act), row_bytes, static_cast<const uint8_t*>(blob), M,
               N, K, y, pl.ngl, s_lo, k_hi, accum ? 1 : 0, out_bf16 ? 1 : 0, nullptr, 64, nullptr, 0, M, 1,
               pl.ks, pl.ss, cnt, part};
    const bool single = num_groups(N) <= pl.grid / pl.ks;     // one group per workgroup
    if (fmt == kNV) return launch_fmt<kNV>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s, single);
    return launch_fmt<kMX>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s, single);
}

hipError_t launch_gemm_grouped(int fmt, const GemmPlan& pl, bool comp, const void* act, int64_t row_bytes,
                               int M_total, const void* blobs, int64_t blob_stride, int E, const int32_t* offsets,
                               int max_rows, int64_t N, int64_t K, float* y, hipStream_t s) {
    if (pl.ks != 1) return hipErrorInvalidValue;
    GemmArgs a{static_cast<const uint8_t*>(act), row_bytes, static_cast<const uint8_t*>(blobs), max_rows, N, K, y,
               pl.ngl, 0, K, 0, 0, nullptr, 64, offsets, blob_stride, M_total, E, 1, 0, nullptr, nullptr};
    const bool single = num_groups(N) <= pl.grid;
    if (fmt == kNV) return launch_fmt<kNV>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s, single);
    return launch_fmt<kMX>(a, pl.rt, comp, pl.maxs, pl.kw, pl.grid, s, single);
}

InqPlan plan_gemm_inq(int fmt, int64_t M, int64_t N, int64_t K, bool comp, int num_cus) {
    InqPlan q;
    if (fmt == kNV && comp) return q;                    // not instantiated (the two launches are faster)
    const int64_t S = num_steps(K);
    const int64_t B = comp ? 2 * M : M;
    if (B > 16 || S > 64) return q;                      // one row tile, up to 4 steps per wave
    q.pl = plan_gemm_small(M, N, S, comp, num_cus);
    if (q.pl.rt != 1 || q.pl.maxs > 4) return q;
    q.qrow = (int)((64 * q.pl.kw / M) / 64 * 64);        // threads per row, whole waves
    if (q.qrow < 64) return q;
    const int64_t ncq = (K + 8 * q.qrow - 1) / (8 * q.qrow);
    if (ncq > 4) return q;
    q.ncq = ncq <= 2 ? 2 : 4;
    const int64_t rec = B * act_row_bytes(fmt, K);
    const int64_t per_group = (int64_t)q.pl.kw * (comp ? 512 : 1024);
    const int64_t fit = (kLdsInq - 256 - rec) / per_group;
    if (fit < 1) return q;
    if (q.pl.ngl > fit) q.pl.ngl = (int)fit;
    if (q.pl.ngl > 64) q.pl.ngl = 64;                   // counters within their 256 bytes
    q.ok = true;
    return q;
}

hipError_t launch_gemm_inq(int fmt, const InqPlan& q, bool comp, const void* x, const void* blob, int M, int64_t N,
                           int64_t K, void* y, bool out_bf16, hipStream_t s) {
    if (q.pl.ks != 1) return hipErrorInvalidValue;
    GemmArgs a{nullptr, act_row_bytes(fmt, K), static_cast<const uint8_t*>(blob), M, N, K, y, q.pl.ngl, 0, K, 0,
               out_bf16 ? 1 : 0, x, q.qrow, nullptr, 0, M, 1, 1, 0, nullptr, nullptr};
    const bool single = num_groups(N) <= q.pl.grid;
    if (fmt == kNV) {   // compensated NVFP4 always takes the two-launch path
        if (comp) return hipErrorInvalidValue;
        return launch_inq_fmt<kNV, false>(a, q.pl.maxs, q.ncq, q.pl.kw, q.pl.grid, s, single);
    }
    return comp ? launch_inq_fmt<kMX, true>(a, q.pl.maxs, q.ncq, q.pl.kw, q.pl.grid, s, single)
                : launch_inq_fmt<kMX, false>(a, q.pl.maxs, q.ncq, q.pl.kw, q.pl.grid, s, single);
}

}  // namespace rsfp4
