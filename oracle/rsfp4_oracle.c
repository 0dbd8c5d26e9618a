/*
 * rsfp4_oracle.c -- plain, slow, scalar CPU oracle for the residue-compensated
 * block-scaled FP4 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the tests, the smoke check and the bench's CPU-baseline leg do.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Sources (all from the page "ResServe: Accurate and Efficient FP4 LLM Inference
 * with Residue Compensation", arXiv 2611.08713):
 *   - Section 2 (Background) and Figure 1: E2M1 elements; NVFP4 = 16-element blocks
 *     with an E4M3 block scale and an FP32 tensor scale; MXFP4 = 32-element blocks
 *     with a power-of-two E8M0 scale and no tensor scale.
 *   - Appendix B.2, Eqs. 8-10: Max_i = max|x| over block i, s_i = Max_i / 6,
 *     alpha = max_i s_i / 448, s_i,FP8 = round_E4M3(s_i / alpha),
 *     s~_i = alpha * s_i,FP8, x_FP4 = round_E2M1(x / s~_i), x^ = s~_i * x_FP4.
 *   - Section 2 (QDQ notation): the residue is r = x - QDQ(x).
 *   - Section 4.2, Eq. 1 and Section 4.3, Eq. 2: Y = X^ W^ + R^ W^ (full residue),
 *     formed as the stacked product [X^; R^] W^ and the Fold Y_j = Z_j + Z_{M+j}.
 *
 * Readings taken where the page leaves a step open (each one is listed with its
 * reason in the design notes of the repository):
 *   - the tensor scale is computed as amax / 2688 (2688 = 6 * 448), per row for
 *     activations and for the residue, per tensor for weights;
 *   - the block scale argument is t = blockmax / (6 * s_g) (product first);
 *   - elements are q = v / s~ (IEEE division), dequantization is fl(s~ * e);
 *   - E4M3 is the FN variant: saturates to 448, never emits the NaN code 0x7F;
 *     a NaN or non-positive argument encodes to 0x00;
 *   - an element whose effective scale s~ is zero gets magnitude code 0;
 *   - the sign bit of every code is copied from the input (so -tiny -> 0x8);
 *   - MXFP4 block scale is 2^(floor(log2(blockmax)) - 2), clamped to the E8M0
 *     range [2^-127, 2^127]; an all-zero block gets byte 0x00;
 *   - nibble order: the element with the even K index sits in the low nibble.
 *
 * Selective compensation (K-Ext; ResServe Section 5.2 "Selective Prefill
 * Execution", Eq. 6, Appendix B.1 Eq. 7, Figure 15), in the reading listed in
 * the design notes:
 *   - calibration statistic of channel i: the sum over calibration rows of |x|
 *     in binary64, rows in order (comparing sums is comparing means);
 *   - per 8-channel group, the k channels with the largest statistic; ties go
 *     to the lower channel index; an 8-bit mask per group records them;
 *   - the extension holds the selected residues group by group, each group's
 *     channels in increasing order, K_eff = K + (K/8) k;
 *   - the extension is quantized in its own 16 (NVFP4) / 32 (MXFP4) blocks;
 *     NVFP4 uses the base row's tensor scale for them (an extended row carries
 *     one tensor scale in the GEMM), MXFP4 its E8M0 rule;
 *   - the weights gain the selected columns in the same order and are quantized
 *     as one K_eff-wide matrix (same per-tensor scale, the columns repeat).
 *
 * Arithmetic: every quantization step is IEEE binary32 with round-to-nearest-even;
 * this file is compiled with -ffp-contract=off so no multiply-add is fused.
 * The linear accumulates exact fp32 x fp32 products in binary64.
 *
 * The encoders are written as exhaustive nearest-value searches over the code
 * tables (not as bit manipulation), so they stay independent of any fast encoder.
 */
#ifdef _OPENMP
#include <omp.h>
#endif
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ---------------------------------------------------------------- E2M1 ---- */

/* The eight non-negative E2M1 magnitudes, indexed by the 3-bit magnitude code
 * (ResServe, Section 2 / Figure 1: 1 sign bit, 2 exponent bits, 1 mantissa bit,
 * largest magnitude 6). */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

ORACLE_API float oracle_e2m1_value(uint8_t code) {
    float m = E2M1_MAG[code & 7u];
    return (code & 8u) ? -m : m;
}

/* Nearest E2M1 magnitude to u >= 0; on an exact tie the even code wins; anything
 * above 6 saturates to 6; NaN encodes to 0. Exhaustive search over 8 values. */
ORACLE_API uint8_t oracle_e2m1_encode_mag(float u) {
    if (!(u == u)) return 0;
    if (u > 6.0f) return 7;
    uint8_t best = 0;
    double best_d = fabs((double)u - (double)E2M1_MAG[0]);
    for (uint8_t c = 1; c < 8; ++c) {
        double d = fabs((double)u - (double)E2M1_MAG[c]);
        if (d < best_d || (d == best_d && (c & 1u) == 0 && (best & 1u) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* ---------------------------------------------------------------- E4M3 ---- */

/* E4M3 (FN) decode: 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN. Subnormals are m * 2^-9. Written from the format definition. */
ORACLE_API float oracle_e4m3_value(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* Nearest non-negative finite E4M3 value to t (codes 0x00..0x7E); ties go to the
 * even code; t above 448 saturates to 448 (0x7E); NaN and t <= 0 give 0x00.
 * Exhaustive search over the 127 candidate codes. */
static float e4m3_table[0x7F];
static int e4m3_table_ready = 0;

ORACLE_API uint8_t oracle_e4m3_encode(float t) {
    if (!(t > 0.0f)) return 0;
    if (t >= 448.0f) return 0x7E;
    if (!e4m3_table_ready) { /* decoded values of codes 0x00..0x7E, filled once */
        for (int c = 0; c <= 0x7E; ++c) e4m3_table[c] = oracle_e4m3_value((uint8_t)c);
        e4m3_table_ready = 1;
    }
    uint8_t best = 0;
    double best_d = fabs((double)t);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)t - (double)e4m3_table[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1u) == 1)) {
            best = (uint8_t)c;
            best_d = d;
        }
    }
    return best;
}

/* ---------------------------------------------------------------- E8M0 ---- */

/* MXFP4 block scale byte for a block whose largest magnitude is a (a >= 0):
 * the scale is 2^(floor(log2 a) - 2), stored as the biased exponent (bias 127),
 * clamped to [-127, 127]; a == 0 gives 0x00. floor(log2 a) comes from frexp,
 * which is exact for every finite binary32 value including subnormals. */
ORACLE_API uint8_t oracle_e8m0_for_amax(float a) {
    if (!(a > 0.0f)) return 0;
    int ex;
    (void)frexp((double)a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return (uint8_t)(e + 127);
}

ORACLE_API float oracle_e8m0_value(uint8_t b) {
    return (float)ldexp(1.0, (int)b - 127);
}

/* ------------------------------------------------------- NVFP4 rows ---- */

/* Tensor (global) scale from an absolute maximum: amax / (6 * 448). */
ORACLE_API float oracle_nvfp4_global_scale(float amax) {
    return amax / 2688.0f;
}

ORACLE_API float oracle_absmax(const float* v, int64_t n) {
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float u = fabsf(v[i]);
        if (u > a) a = u;
    }
    return a;
}

/* Quantize one row of K values (K a multiple of 16) with a given tensor scale s_g
 * (Appendix B.2, Eqs. 8-10, in the reading above).
 * codes: K/2 bytes (low nibble = even index); scales: K/16 E4M3 bytes;
 * deq (optional): the K dequantized values fl(s~ * e). */
ORACLE_API void oracle_nvfp4_quantize_row(const float* v, int64_t K, float s_g,
                                          uint8_t* codes, uint8_t* scales, float* deq) {
    for (int64_t b = 0; b < K / 16; ++b) {
        const float* blk = v + 16 * b;
        float amax_b = oracle_absmax(blk, 16);
        float t = amax_b / (6.0f * s_g);
        uint8_t sb = oracle_e4m3_encode(t);
        float S_b = oracle_e4m3_value(sb);
        float st = S_b * s_g; /* effective scale s~ */
        scales[b] = sb;
        for (int j = 0; j < 16; ++j) {
            float x = blk[j];
            uint8_t mag = 0;
            if (st != 0.0f) {
                float q = x / st;
                mag = oracle_e2m1_encode_mag(fabsf(q));
            }
            uint8_t code = (uint8_t)((signbit(x) ? 8u : 0u) | mag);
            int64_t k = 16 * b + j;
            if ((k & 1) == 0)
                codes[k / 2] = code;
            else
                codes[k / 2] = (uint8_t)(codes[k / 2] | (code << 4));
            if (deq) deq[k] = st * oracle_e2m1_value(code);
        }
    }
}

/* ------------------------------------------------------- MXFP4 rows ---- */

/* Quantize one row of K values (K a multiple of 32): per 32-block E8M0 scale X,
 * elements q = v / X rounded to E2M1 (saturating at 6); deq = X * e. */
ORACLE_API void oracle_mxfp4_quantize_row(const float* v, int64_t K,
                                          uint8_t* codes, uint8_t* scales, float* deq) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const float* blk = v + 32 * b;
        float amax_b = oracle_absmax(blk, 32);
        uint8_t e8 = oracle_e8m0_for_amax(amax_b);
        float X = oracle_e8m0_value(e8);
        scales[b] = e8;
        for (int j = 0; j < 32; ++j) {
            float x = blk[j];
            float q = x / X;
            uint8_t mag = oracle_e2m1_encode_mag(fabsf(q));
            uint8_t code = (uint8_t)((signbit(x) ? 8u : 0u) | mag);
            int64_t k = 32 * b + j;
            if ((k & 1) == 0)
                codes[k / 2] = code;
            else
                codes[k / 2] = (uint8_t)(codes[k / 2] | (code << 4));
            if (deq) deq[k] = X * oracle_e2m1_value(code);
        }
    }
}

/* ------------------------------------------- activations with residue ---- */

/* Quantize M activation rows; with_residue != 0 also forms r = x - deq(q(x)) in
 * fp32 and quantizes it "the same way" (its own per-row tensor scale for NVFP4).
 * Output rows are stacked [X^; R^]: rows 0..M-1 base, rows M..2M-1 residue.
 * fmt: 0 = NVFP4, 1 = MXFP4.
 * codes: R x K/2; scales: R x K/blk; globals: R floats (NVFP4; zeros for MXFP4);
 * deq: R x K floats (optional); resid: M x K floats (optional; the fp32 residue). */
ORACLE_API void oracle_quantize_act(int fmt, const float* x, int64_t M, int64_t K,
                                    int with_residue, uint8_t* codes, uint8_t* scales,
                                    float* globals, float* deq, float* resid) {
    int64_t blk = fmt == 0 ? 16 : 32;
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * K;
        float* drow = deq ? deq + m * K : (float*)0;
        if (fmt == 0) {
            float sg = oracle_nvfp4_global_scale(oracle_absmax(row, K));
            globals[m] = sg;
            oracle_nvfp4_quantize_row(row, K, sg, codes + m * (K / 2), scales + m * (K / blk), drow);
        } else {
            globals[m] = 0.0f;
            oracle_mxfp4_quantize_row(row, K, codes + m * (K / 2), scales + m * (K / blk), drow);
        }
    }
    if (!with_residue) return;
    /* residue r = x - deq(q(x)): the dequantized base is rebuilt from the stored
     * codes and scales with the same association, fl(fl(S_b * s_g) * e) */
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * K;
        float* r = resid + m * K;
        const uint8_t* c = codes + m * (K / 2);
        const uint8_t* s = scales + m * (K / blk);
        for (int64_t k = 0; k < K; ++k) {
            uint8_t code = (uint8_t)((k & 1) ? (c[k / 2] >> 4) : (c[k / 2] & 15u));
            float e = oracle_e2m1_value(code);
            float dk;
            if (fmt == 0)
                dk = (oracle_e4m3_value(s[k / 16]) * globals[m]) * e;
            else
                dk = oracle_e8m0_value(s[k / 32]) * e;
            r[k] = row[k] - dk;
        }
        int64_t rr = M + m;
        float* drow = deq ? deq + rr * K : (float*)0;
        if (fmt == 0) {
            float sg = oracle_nvfp4_global_scale(oracle_absmax(r, K));
            globals[rr] = sg;
            oracle_nvfp4_quantize_row(r, K, sg, codes + rr * (K / 2), scales + rr * (K / blk), drow);
        } else {
            globals[rr] = 0.0f;
            oracle_mxfp4_quantize_row(r, K, codes + rr * (K / 2), scales + rr * (K / blk), drow);
        }
    }
}

/* ----------------------------------------------------------- weights ---- */

/* Quantize nrows weight rows of length K. NVFP4 uses the given per-tensor scale
 * s_gw (from the absolute maximum over the whole tensor); MXFP4 ignores it. */
ORACLE_API void oracle_quantize_weight_rows(int fmt, const float* W, int64_t nrows, int64_t K,
                                            float s_gw, uint8_t* codes, uint8_t* scales,
                                            float* deq) {
    int64_t blk = fmt == 0 ? 16 : 32;
    /* rows are independent given the tensor scale (threads: timing build only) */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < nrows; ++n) {
        float* drow = deq ? deq + n * K : (float*)0;
        if (fmt == 0)
            oracle_nvfp4_quantize_row(W + n * K, K, s_gw, codes + n * (K / 2), scales + n * (K / blk), drow);
        else
            oracle_mxfp4_quantize_row(W + n * K, K, codes + n * (K / 2), scales + n * (K / blk), drow);
    }
}

/* ------------------------------------------------------------ linear ---- */

/* y[m, n] = sum_k dx[m, k] * dw[n, k] (+ sum_k dr[m, k] * dw[n, k] when
 * compensated), accumulated in binary64 over exact fp32 x fp32 products.
 * dx holds the stacked dequantized activation rows: rows 0..M-1 base and, when
 * compensated, rows M..2M-1 residue (Eq. 2's [X^; R^] with the Fold).
 * beta[m, n] = sum_k |dx dw| (+ |dr dw|): the scale of the rounding bound. */
ORACLE_API void oracle_linear(const float* dx, const float* dw, int64_t M, int64_t N, int64_t K,
                              int compensated, double* y, double* beta) {
    for (int64_t m = 0; m < M; ++m) {
        const float* xb = dx + m * K;
        const float* xr = compensated ? dx + (M + m) * K : (const float*)0;
        /* Every output is its own sum, so the channels may be spread over
         * threads (only the timing build enables OpenMP; results are the
         * same bits either way). */
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            const float* w = dw + n * K;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)xb[k] * (double)w[k];
                acc += p;
                mag += fabs(p);
            }
            if (xr) {
                for (int64_t k = 0; k < K; ++k) {
                    double p = (double)xr[k] * (double)w[k];
                    acc += p;
                    mag += fabs(p);
                }
            }
            y[m * N + n] = acc;
            if (beta) beta[m * N + n] = mag;
        }
    }
}

/* ----------------------------------------- selective compensation (K-Ext) ---- */

/* Calibration statistic (Appendix B.1): sum[i] += |x[t, i]| for t = 0 .. T-1 in
 * binary64, one row after another.  The page scores a channel by its mean
 * absolute activation; for a fixed number of rows the sum orders channels the
 * same way.  Continuing from an earlier sum is the same as summing the
 * concatenated rows in order. */
ORACLE_API void oracle_channel_abs_sum(const float* x, int64_t T, int64_t K, double* sum) {
    for (int64_t t = 0; t < T; ++t)
        for (int64_t i = 0; i < K; ++i) sum[i] += fabs((double)x[t * K + i]);
}

/* Block-local selection (Appendix B.1, Eq. 7): in every group of 8 channels the
 * k with the largest score, ties to the lower index.  masks: K/8 bytes, bit j
 * set when channel 8g + j is selected. */
ORACLE_API void oracle_kext_select(const double* score, int64_t K, int k, uint8_t* masks) {
    for (int64_t g = 0; g < K / 8; ++g) {
        const double* s = score + 8 * g;
        uint8_t mask = 0;
        for (int q = 0; q < k; ++q) {      /* take the best channel not yet taken, k times */
            int best = -1;
            for (int j = 0; j < 8; ++j) {
                if (mask & (1u << j)) continue;
                if (best < 0 || s[j] > s[best]) best = j;   /* strict: lower index wins ties */
            }
            mask = (uint8_t)(mask | (1u << best));
        }
        masks[g] = mask;
    }
}

/* Extension order (Section 5.3, Eq. 6 and Appendix B.1): extension element p
 * belongs to group p / k and is the (p % k)-th selected channel of that group in
 * increasing channel order.  Returns the channel index; masks must hold exactly
 * k bits per byte. */
static int64_t kext_channel(const uint8_t* masks, int k, int64_t p) {
    const int64_t g = p / k;
    int want = (int)(p % k);
    for (int j = 0; j < 8; ++j) {
        if (!(masks[g] & (1u << j))) continue;
        if (want == 0) return 8 * g + j;
        --want;
    }
    return -1;
}

/* Extended weight (Eq. 6): Wext[n] = [W[n, 0..K) | W[n, S]] with the selected
 * columns in extension order; K_eff = K + (K/8) k.  Quantizing Wext as one
 * K_eff-wide tensor gives the page's W^_S in the extended block layout. */
ORACLE_API void oracle_kext_extend_weight(const float* W, int64_t N, int64_t K, const uint8_t* masks,
                                          int k, float* Wext) {
    const int64_t ext = (K / 8) * k, KE = K + ext;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t i = 0; i < K; ++i) Wext[n * KE + i] = W[n * K + i];
        for (int64_t p = 0; p < ext; ++p) Wext[n * KE + K + p] = W[n * K + kext_channel(masks, k, p)];
    }
}

/* Quantize M rows into K-Ext records of K_eff = K + (K/8) k elements (Eq. 6;
 * Appendix B.2, Algorithm 1): elements [0, K) are the base q(x) exactly as in
 * oracle_quantize_act; elements [K, K_eff) are the residues r = x - deq(q(x))
 * of the selected channels in extension order, quantized in their own blocks
 * (NVFP4: with the base row's tensor scale, which the algorithm passes to both
 * block-scale steps; MXFP4: the E8M0 rule).  codes: M x K_eff/2; scales:
 * M x K_eff/blk; globals: M (NVFP4 base tensor scale, 0 for MXFP4); deq:
 * M x K_eff or NULL; work: (K/8) k floats of scratch. */
ORACLE_API void oracle_kext_quantize_act(int fmt, const float* x, int64_t M, int64_t K,
                                         const uint8_t* masks, int k, uint8_t* codes, uint8_t* scales,
                                         float* globals, float* deq, float* work) {
    const int64_t blk = fmt == 0 ? 16 : 32;
    const int64_t ext = (K / 8) * k, KE = K + ext;
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * K;
        uint8_t* c = codes + m * (KE / 2);
        uint8_t* s = scales + m * (KE / blk);
        float* d = deq ? deq + m * KE : (float*)0;
        float sg = 0.0f;
        if (fmt == 0) {
            sg = oracle_nvfp4_global_scale(oracle_absmax(row, K));
            oracle_nvfp4_quantize_row(row, K, sg, c, s, d);
        } else {
            oracle_mxfp4_quantize_row(row, K, c, s, d);
        }
        globals[m] = sg;
        for (int64_t p = 0; p < ext; ++p) {
            const int64_t i = kext_channel(masks, k, p);
            const uint8_t code = (uint8_t)((i & 1) ? (c[i / 2] >> 4) : (c[i / 2] & 15u));
            const float e = oracle_e2m1_value(code);
            const float st = fmt == 0 ? oracle_e4m3_value(s[i / 16]) * sg : oracle_e8m0_value(s[i / 32]);
            work[p] = row[i] - st * e;
        }
        if (fmt == 0)
            oracle_nvfp4_quantize_row(work, ext, sg, c + K / 2, s + K / blk, d ? d + K : (float*)0);
        else
            oracle_mxfp4_quantize_row(work, ext, c + K / 2, s + K / blk, d ? d + K : (float*)0);
    }
}

/* ------------------------------- paper numerics (static tensor scale) ---- */
/* The operator as the page's fused quantizer computes it (Appendix B.2: Eq. 8
 * and the pack8 description, Algorithm 1), in the reading listed in the design
 * notes, NVFP4 only:
 *   - one tensor scale alpha per activation tensor, an input (static or
 *     calibrated); when derived from the data, alpha = (amax / 6) / 448 with
 *     both divisions rounded (Eq. 8: s_i = Max_i / 6, alpha = max_i s_i / 448);
 *   - block scale byte E4M3_RNE((Max_i / 6) / alpha), both divisions rounded;
 *   - the multiplier scale = 1 / (alpha * S_b) (0 when alpha * S_b is 0); the
 *     element code is E2M1_RNE(x * scale);
 *   - the residue r = x - e / scale (x when scale is 0): the decoded code is
 *     rescaled by dividing by the multiplier;
 *   - the residue shares alpha and is quantized by the same steps.
 * The dequantized value the product uses is fl(alpha * S_b) * e. */

/* alpha = fl(fl(amax / 6) / 448) over n values. */
ORACLE_API float oracle_nvfp4_alpha(const float* x, int64_t n) {
    const float s = oracle_absmax(x, n) / 6.0f;
    return s / 448.0f;
}

/* One row with tensor scale alpha.  codes K/2, scales K/16, deq K (optional),
 * resid K (optional: the residue as the algorithm forms it). */
ORACLE_API void oracle_nvfp4_quantize_row_alg1(const float* v, int64_t K, float alpha, uint8_t* codes,
                                               uint8_t* scales, float* deq, float* resid) {
    for (int64_t b = 0; b < K / 16; ++b) {
        const float* blk = v + 16 * b;
        const float s = oracle_absmax(blk, 16) / 6.0f;
        const uint8_t sb = oracle_e4m3_encode(s / alpha);
        const float st = alpha * oracle_e4m3_value(sb);
        const float mult = st > 0.0f ? 1.0f / st : 0.0f;
        scales[b] = sb;
        for (int j = 0; j < 16; ++j) {
            const float x = blk[j];
            const float u = x * mult;
            const uint8_t code = (uint8_t)((signbit(x) ? 8u : 0u) | oracle_e2m1_encode_mag(fabsf(u)));
            const int64_t k = 16 * b + j;
            if ((k & 1) == 0)
                codes[k / 2] = code;
            else
                codes[k / 2] = (uint8_t)(codes[k / 2] | (code << 4));
            const float e = oracle_e2m1_value(code);
            if (deq) deq[k] = st * e;
            if (resid) resid[k] = mult > 0.0f ? x - e / mult : x;
        }
    }
}

/* M rows (and, with_residue, their residues as rows M..2M-1) with one tensor
 * scale alpha for all of them.  Layout as oracle_quantize_act; globals = alpha;
 * resid: M x K (optional). */
ORACLE_API void oracle_quantize_act_alg1(const float* x, int64_t M, int64_t K, float alpha, int with_residue,
                                         uint8_t* codes, uint8_t* scales, float* globals, float* deq,
                                         float* resid, float* work) {
    for (int64_t m = 0; m < M; ++m) {
        float* r = with_residue ? (resid ? resid + m * K : work) : (float*)0;
        oracle_nvfp4_quantize_row_alg1(x + m * K, K, alpha, codes + m * (K / 2), scales + m * (K / 16),
                                       deq ? deq + m * K : (float*)0, r);
        globals[m] = alpha;
        if (!with_residue) continue;
        const int64_t rr = M + m;
        oracle_nvfp4_quantize_row_alg1(r, K, alpha, codes + rr * (K / 2), scales + rr * (K / 16),
                                       deq ? deq + rr * K : (float*)0, (float*)0);
        globals[rr] = alpha;
    }
}

/* ------------------------------------------- decode attention (ResAttn) ---- */
/* ResServe Section 4.3 (Eq. 3) and Section 5.2 "ResAttn Execution": for the
 * query heads sharing one KV head, the scores are Q^ K^T + R^ K^T (base and
 * quantized residue of each query row against the NVFP4 keys), scaled, folded
 * before the softmax; the output is softmax(S) V^ with V^ the dequantized
 * NVFP4 values.  Here in binary64 from dequantized operands:
 *   qb, qr: [H_q, d] dequantized query base / residue rows of one sequence
 *           (qr NULL: the uncompensated scores Q^ K^T);
 *   kd, vd: [L, H_kv, d] dequantized keys / values of its L cached tokens;
 *   out:    [H_q, d].  Query head h reads KV head h / (H_q / H_kv).
 * score_t = sm_scale * sum_i (qb_i + qr_i) k_ti, with every product exact in
 * binary64; p_t = exp(score_t - max_t score_t); out = sum_t p_t v_t / sum_t p_t. */
ORACLE_API void oracle_attention_decode(const float* qb, const float* qr, const float* kd, const float* vd,
                                        int64_t L, int64_t H_q, int64_t H_kv, int64_t d, double sm_scale,
                                        double* out, double* work) {
    const int64_t G = H_q / H_kv;
    double* s = work;                         /* L scores */
    for (int64_t h = 0; h < H_q; ++h) {
        const int64_t hk = h / G;
        double mx = -INFINITY;
        for (int64_t t = 0; t < L; ++t) {
            const float* k = kd + (t * H_kv + hk) * d;
            double acc = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                acc += (double)qb[h * d + i] * (double)k[i];
                if (qr) acc += (double)qr[h * d + i] * (double)k[i];
            }
            s[t] = sm_scale * acc;
            if (s[t] > mx) mx = s[t];
        }
        double den = 0.0;
        for (int64_t i = 0; i < d; ++i) out[h * d + i] = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double p = exp(s[t] - mx);
            den += p;
            const float* v = vd + (t * H_kv + hk) * d;
            for (int64_t i = 0; i < d; ++i) out[h * d + i] += p * (double)v[i];
        }
        for (int64_t i = 0; i < d; ++i) out[h * d + i] /= den;
    }
}

/* Threads the OpenMP timing build runs its parallel loops with (1 in the
 * plain build). */
ORACLE_API int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
