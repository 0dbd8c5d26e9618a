/*
 * rsfp4.h -- C ABI of the residue-compensated block-scaled FP4 linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the full-residue decode linear of the page "ResServe: Accurate
 * and Efficient FP4 LLM Inference with Residue Compensation" (arXiv 2611.08713):
 *   - activations x[M,K] are quantized at run time to NVFP4 or MXFP4 (Section 2,
 *     Figure 1; NVFP4 scale rules of Appendix B.2, Eqs. 8-10);
 *   - the residue r = x - deq(q(x)) is formed in registers and quantized the same
 *     way (Section 2; Section 4.4: residue generation fused into the quantizer);
 *   - weights are quantized and laid out once, offline (Figure 1c; Section 5.4:
 *     weight preparation happens once during export);
 *   - the compensated product y = deq(q(x)) W^T + deq(q(r)) W^T is the stacked
 *     GEMM [X^; R^] W^T whose paired rows are added on chip (Section 4.2, Eq. 1;
 *     Section 4.3, Eq. 2, the Fold), reading each weight tile once.
 *
 * Numerics (both formats): E2M1 elements rounded to nearest, ties to even,
 * saturated at +-6; the element with the even K index sits in the low nibble.
 *   NVFP4: 16-element blocks, E4M3 (FN) block scale, fp32 tensor scale
 *     s_g = amax / 2688 (per row for x and for r, per tensor for W);
 *     block byte = E4M3_RNE(blockmax / (6 * s_g)) saturated at 448 (0x7e);
 *     element = E2M1_RNE(v / (S_b * s_g)); value = (S_b * s_g) * e.
 *   MXFP4: 32-element blocks, E8M0 scale 2^(floor(log2 blockmax) - 2) clamped to
 *     [2^-127, 2^127] (byte 0 for an all-zero block), no tensor scale;
 *     element = E2M1_RNE(v / X); value = X * e.
 *   The output y is fp32 (the *_bf16 linears: bf16, rounded to nearest even
 *   from the fp32 result), accumulated in fp32 on the matrix cores.
 *   NaN or infinite inputs give unspecified codes and outputs.
 *   The paper-numerics NVFP4 quantizer (rsfp4_nvfp4_quantize_act_alpha) takes
 *   a tensor scale alpha instead and follows the page's fused quantizer; see
 *   its comment.
 *
 * Conventions for every call:
 *   - Pointers named W, x, act, w_packed, y, codes, scales, s_g are DEVICE
 *     pointers owned by the caller; the library allocates no device memory and
 *     keeps no device state besides its code objects.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call only enqueues work on it and returns; nothing synchronizes except
 *     where a call says so.
 *   - Arguments are validated on the host before anything is enqueued. A failed
 *     check returns a status other than RSFP4_OK, enqueues nothing, and leaves
 *     a message for rsfp4_last_error() (per thread). A HIP launch failure returns
 *     RSFP4_ERR_HIP with the HIP error string in the message.
 *   - Shape limits: M >= 1, N >= 1, K >= 32 and K % 32 == 0 (both formats, so a
 *     K-run of 32 is whole in either block size); M <= 65535; quantize needs
 *     K <= 32768; the linear needs K <= 32768 and N <= 2^24, and where it runs
 *     the tiled kernel (more than 32 operand rows) an activation operand below
 *     2^31 bytes.  Calls outside these limits return RSFP4_ERR_SHAPE or
 *     RSFP4_ERR_UNSUPPORTED.
 *   - All calls are thread-safe; concurrent calls on different streams are
 *     independent.
 */
#ifndef RSFP4_H
#define RSFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSFP4_ABI_VERSION 1

typedef enum { RSFP4_NVFP4 = 0, RSFP4_MXFP4 = 1 } rsfp4_format;
typedef enum { RSFP4_F32 = 0, RSFP4_BF16 = 1 } rsfp4_dtype;

typedef enum {
    RSFP4_OK = 0,
    RSFP4_ERR_NULL = 1,             /* a required pointer is NULL */
    RSFP4_ERR_SHAPE = 2,            /* M, N or K outside the documented limits */
    RSFP4_ERR_ALIGN = 3,            /* a buffer is not 16-byte aligned */
    RSFP4_ERR_FORMAT = 4,           /* unknown format or dtype */
    RSFP4_ERR_BUFFER_TOO_SMALL = 5, /* a byte count is below the size query */
    RSFP4_ERR_UNSUPPORTED = 6,      /* valid request this build does not run */
    RSFP4_ERR_HIP = 7               /* the HIP runtime reported an error */
} rsfp4_status;

/* Version of this ABI (RSFP4_ABI_VERSION of the built library). */
int rsfp4_abi_version(void);
/* Static string naming a status code; never NULL. */
const char* rsfp4_status_string(int status);
/* Detail of the last failed call on this thread ("" if none); valid until the
 * next call on the same thread. */
const char* rsfp4_last_error(void);

/* ------------------------------------------------------------------ sizes --
 * Activation buffer ("act"): one record per quantized row, rows stacked as in
 * Eq. 2 of the ResServe page: rows 0..M-1 hold q(x), rows M..2M-1 hold q(r)
 * (present when quantized with_residue).  Record layout, stride
 * rsfp4_act_row_bytes(fmt, K) (a multiple of 16):
 *   [0, 4)              fp32 tensor scale s_g of the row (NVFP4; 0 for MXFP4)
 *   [4, 16)             zero
 *   [16, 16 + K/2)      E2M1 codes, element 2j in the low nibble of byte j
 *   [16 + K/2, +K/blk)  block scale bytes (E4M3 for NVFP4, E8M0 for MXFP4)
 *   then padding to the stride, left unwritten (unspecified).
 * The first M records of a with_residue buffer form a valid plain buffer. */
size_t rsfp4_act_row_bytes(int fmt, int64_t K);
size_t rsfp4_packed_act_bytes(int fmt, int64_t M, int64_t K, int with_residue);

/* Packed weight blob: a 256-byte header (magic "RSF4", ABI version, format, N,
 * K, the NVFP4 per-tensor scale) followed by ceil(N/16) groups of 16 output
 * channels; each group holds ceil(K/512) quads of four 128-element K steps.  A
 * quad is 4 x 1024 bytes of codes, each 1 KB laid out for one 64-lane wave load
 * (lane l = 16*g + i holds channel i, K-elements 32*g .. 32*g+31 of the step),
 * followed by the quad's block scales with each lane's four steps adjacent
 * (NVFP4: 8 bytes per lane, the E4M3 bytes of blocks 2g, 2g+1 per step; MXFP4:
 * 4 bytes per lane, the E8M0 byte of block g per step).  Channels beyond N,
 * K-elements beyond K and the padding steps of the last quad are zero codes
 * with zero scales.  Only rsfp4_unpack_weights_canonical reads it back. */
size_t rsfp4_packed_weight_bytes(int fmt, int64_t N, int64_t K);

/* Device workspace (bytes) with which a linear call of this shape may split K
 * across workgroups; 0 when its plan does not split.  The value depends on the
 * current device's compute-unit count.  Shapes that split (compensated NVFP4,
 * K <= 16384 on the narrow kernel: with at most 16 operand rows when there are
 * few 16-channel groups (at most one per compute unit) and K of 64 and more
 * steps of 128 -- the ResServe page's tile-count model, Section 5.1 Eq. 5:
 * too few units of work leave compute units idle -- and with 17..32 operand
 * rows when K of more than 32 steps of 128 divides into 2..4 equal slices of
 * at most 32 steps, one pass over K instead of launches of 32 steps) sum
 * their K slices' partial outputs
 * through the workspace: 4096 int counters, one per 16-channel group (the first 16384
 * bytes; only N of at most 4096 groups splits), then one partial-sum record
 * per group and slice.  The counters must be zero before the workspace's
 * first use (e.g. allocate it zero-filled); every call leaves them zero
 * again, so one workspace serves any number of calls of any shapes in stream
 * order (calls that may run concurrently need workspaces of their own).  The slices' partials are
 * summed in slice order, so the result does not depend on timing.  A linear
 * call given a NULL or smaller workspace runs the plan without the split
 * (same result up to the summation order of the slices).  Wide operands, more
 * than 32 operand rows B (2M compensated, M plain), use the workspace
 * differently (except compensated NVFP4 with 33..64 rows, N <= 4096 and
 * K <= 4096, which runs the narrow kernel): after the same 16384-byte counter
 * area (left zero) the call rewrites the activation records in tiles of
 * 16 operand rows, base and residue rows interleaved -- MXFP4 in the
 * packed-weight layout (4352 bytes per tile and quad of 4 steps: 16384 +
 * ceil(B/16) * ceil(K/512) * 4352 bytes in all), NVFP4 as the exact f16
 * products e * S_b in MFMA fragment order (4096 bytes per tile and step of 128:
 * 16384 + ceil(B/16) * ceil(K/128) * 4096 bytes) -- so that the activations
 * stream into LDS as contiguous 1 KB requests.  Given a NULL or smaller
 * workspace the call multiplies the records directly, with the same bits.
 * An NVFP4 product's tiles are 64 rows up to 64 operand rows and from 97
 * to 128 (and up to 256 below N = 16384), else 128, by 32 channels per wave, W = 4 waves (W = 8
 * from N = 16384 on).  With few
 * tiles (while twice the tiles stay within the compute units, K holds at
 * least 16 steps per slice pair and tiles x W is at most 4096) it splits K
 * into ks = 2..8 slices of a multiple of 8 steps: its workspace adds, at the
 * next 256-byte boundary after the rewritten operand, one record of folded
 * partial sums per tile, wave and slice (the tile's rows / 16 x 2 x 64 x
 * 2 floats compensated, one per token of each row pair, x 4 plain),
 * and W counters per tile in the counter area count the slices in and are
 * left zero; the slices are summed in slice order.  With a workspace that
 * holds the rewritten operand but not the partials the product runs unsplit
 * (the same result up to the summation order of the slices).  Without a
 * device to count compute units on the size is the unsplit one.  Wide shapes
 * whose rewritten operand would exceed 1 GiB size to 0 (no rewrite).  ws
 * must be 256-byte aligned. */
size_t rsfp4_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int compensated);

/* ------------------------------------------------------------- prepack ----
 * Quantize W[N,K] (row-major, dtype wt: RSFP4_F32 or RSFP4_BF16) once, offline,
 * into the packed blob at w_packed (w_packed_bytes >= rsfp4_packed_weight_bytes,
 * 256-byte aligned).  NVFP4 takes one tensor scale from max|W| over the whole
 * tensor (ResServe Appendix B.2, Eq. 8 with a per-tensor alpha); MXFP4 scales
 * each 32-block (Section 2).  Enqueues three kernels; W may be freed once the
 * stream has passed them. */
rsfp4_status rsfp4_nvfp4_prepack_weights(const void* W, int wt, int64_t N, int64_t K,
                                         void* w_packed, size_t w_packed_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_prepack_weights(const void* W, int wt, int64_t N, int64_t K,
                                         void* w_packed, size_t w_packed_bytes, void* stream);

/* ------------------------------------------------------------ quantize ----
 * Quantize x[M,K] (row-major, dtype xt) to the activation buffer act
 * (act_bytes >= rsfp4_packed_act_bytes(fmt, M, K, with_residue), 16-byte
 * aligned).  One pass per row: row amax, tensor scale, block scales, codes;
 * with_residue != 0 also forms r = x - deq(q(x)) in fp32 registers and quantizes
 * it with its own row amax (ResServe Section 4.4 and Appendix B.2, Algorithm 1:
 * residue and base produced in the same pass). */
rsfp4_status rsfp4_nvfp4_quantize_act_with_residue(const void* x, int xt, int64_t M, int64_t K,
                                                   int with_residue, void* act, size_t act_bytes,
                                                   void* stream);
rsfp4_status rsfp4_mxfp4_quantize_act_with_residue(const void* x, int xt, int64_t M, int64_t K,
                                                   int with_residue, void* act, size_t act_bytes,
                                                   void* stream);

/* -------------------------------------------------------------- linear ----
 * y[M,N] (fp32, row-major, fully overwritten) from a quantized activation
 * buffer and a packed weight blob of the same format and the same N, K.
 *   *_linear:              y = deq(q(x)) W^T                 (B = M rows; the
 *                          buffer may or may not hold residue rows)
 *   *_linear_compensated:  y = deq(q(x)) W^T + deq(q(r)) W^T (B = 2M rows; the
 *                          buffer must have been quantized with_residue)
 * B = M (plain) or 2M (compensated) activation rows enter the product.  Up to
 * 32 rows (compensated NVFP4 with N <= 4096 and K <= 4096: up to 64), each
 * packed weight step is loaded from HBM once and multiplied with all B rows
 * (the narrow-M, memory-bound regime); above that a 2-D tiled kernel covers
 * 128 rows x 128 channels per workgroup (NVFP4: 64 rows up to 64 operand
 * rows and from 97 to 128, up to 256 below N = 16384, and 256 channels from N = 16384 on; each
 * weight tile is then read once per 64 or 128 rows).  Either way base and residue products of one token
 * land in the same lane's accumulators and are added there before the single
 * store (ResServe Section 4.3, Eq. 2 and Section 5.1, Eq. 4).  With up to 32
 * rows and K above 16384 the narrow kernel runs twice, over the two halves of
 * the K steps, the second launch adding its part to y (so y is written, read
 * back and written again).  act_bytes and w_packed_bytes are checked against
 * the size queries.  ws, ws_bytes: the optional workspace of
 * rsfp4_workspace_bytes (NULL, 0 for none; 256-byte aligned, counters zero on
 * first use, left zero); with it, compensated NVFP4 shapes that gain from it
 * split K across workgroups, and wide operands take the tiled product over
 * rewritten activations (same bits as without), NVFP4 with few tiles split
 * across workgroups in K as well. */
rsfp4_status rsfp4_nvfp4_linear(const void* act, size_t act_bytes, const void* w_packed,
                                size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                float* y, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_nvfp4_linear_compensated(const void* act, size_t act_bytes, const void* w_packed,
                                            size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                            float* y, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_linear(const void* act, size_t act_bytes, const void* w_packed,
                                size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                float* y, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_linear_compensated(const void* act, size_t act_bytes, const void* w_packed,
                                            size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                            float* y, void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): the compensated
 * NVFP4 linear of rsfp4_nvfp4_linear_compensated, same arguments but no
 * workspace: the same plan and the same bits as that call given a workspace of
 * min(rsfp4_workspace_bytes, 16384 + 16777216) bytes.
 * Where the plan splits K it uses the library's own scratch, a device array of
 * 16384 + 16777216 bytes on each GPU (held until the process ends; its address
 * is taken, and its counter area cleared on `stream`, by the first call on a
 * device).  Wide operands (more than 32 operand rows, except 33..64 with N
 * and K at most 4096) use the scratch for their rewritten activations and a
 * split's partial sums as far as they fit in it: a split that does not fit
 * runs unsplit, and rewritten activations that do not fit (more than 16777216
 * bytes: ceil(2M/16) * ceil(K/128) * 4096) are not made (the records path,
 * the same bits as the unsplit tiled product).  It calls no allocator.
 * Narrow shapes whose split would need more than the scratch holds are
 * rejected with RSFP4_ERR_UNSUPPORTED (none of the plans this library makes on
 * a 256-CU device does).  Every call on a GPU shares that GPU's scratch:
 * calls that may overlap on one GPU (other streams, other threads) race;
 * calls in stream order do not. */
rsfp4_status rsfp4_nvfp4_linear_compensated_noalloc(const void* act, size_t act_bytes, const void* w_packed,
                                                    size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                                    float* y, void* stream);

/* ------------------------------------------- bf16 output (the same sums) --
 * As the linears above, with y [M, N] stored as bf16 (uint16 bit patterns,
 * 2-byte aligned): the fp32 Fold result rounded to nearest even, as the
 * page's Fold epilogue writes BF16 (Appendix C.1: linear timing includes the
 * GEMM/Fold to BF16 output).  With up to 32 rows and K above 16384 these run
 * the tiled kernel (one pass over K) instead of two narrow launches. */
rsfp4_status rsfp4_nvfp4_linear_bf16(const void* act, size_t act_bytes, const void* w_packed,
                                     size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, void* y,
                                     void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_nvfp4_linear_compensated_bf16(const void* act, size_t act_bytes, const void* w_packed,
                                                 size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                                 void* y, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_linear_bf16(const void* act, size_t act_bytes, const void* w_packed,
                                     size_t w_packed_bytes, int64_t M, int64_t N, int64_t K, void* y,
                                     void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_linear_compensated_bf16(const void* act, size_t act_bytes, const void* w_packed,
                                                 size_t w_packed_bytes, int64_t M, int64_t N, int64_t K,
                                                 void* y, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------- grouped linear (mixture of experts) --
 * E experts in one launch, the grouped GEMM the ResServe page names as future
 * work for mixture-of-experts models (its conclusion): expert e multiplies
 * the token rows offsets[e] .. offsets[e+1] - 1 of one activation buffer (all
 * tokens quantized together, rows sorted by expert, as the quantize call
 * writes them for M_total rows) by its own packed weights and writes the same
 * rows of y [M_total, N] (fp32); each expert's result is that of the
 * (compensated) linear on its rows alone.
 *   w_packed: E blobs of rsfp4_packed_weight_bytes(fmt, N, K) bytes each, back
 *             to back (each with its own header and tensor scale).
 *   offsets:  DEVICE int32[E + 1], non-decreasing, within [0, M_total] (values
 *             outside are clamped); read by the kernel, so a router on the GPU
 *             can write them without a host round trip.
 *   max_rows: a bound on every expert's row count that the caller guarantees
 *             (it selects the kernel's row tiles): 1 <= max_rows, at most 32
 *             operand rows (max_rows <= 32 plain, <= 16 compensated).  Rows of
 *             an expert past max_rows, and rows of y no expert covers, are left
 *             as they were.
 * K <= 16384 (one narrow launch).  Each expert's channel groups take about
 * num_CUs / E compute units. */
rsfp4_status rsfp4_nvfp4_grouped_linear(const void* act, size_t act_bytes, int64_t M_total, const void* w_packed,
                                        size_t w_packed_bytes, int64_t E, const int32_t* offsets, int64_t max_rows,
                                        int64_t N, int64_t K, float* y, void* stream);
rsfp4_status rsfp4_nvfp4_grouped_linear_compensated(const void* act, size_t act_bytes, int64_t M_total,
                                                    const void* w_packed, size_t w_packed_bytes, int64_t E,
                                                    const int32_t* offsets, int64_t max_rows, int64_t N, int64_t K,
                                                    float* y, void* stream);
rsfp4_status rsfp4_mxfp4_grouped_linear(const void* act, size_t act_bytes, int64_t M_total, const void* w_packed,
                                        size_t w_packed_bytes, int64_t E, const int32_t* offsets, int64_t max_rows,
                                        int64_t N, int64_t K, float* y, void* stream);
rsfp4_status rsfp4_mxfp4_grouped_linear_compensated(const void* act, size_t act_bytes, int64_t M_total,
                                                    const void* w_packed, size_t w_packed_bytes, int64_t E,
                                                    const int32_t* offsets, int64_t max_rows, int64_t N, int64_t K,
                                                    float* y, void* stream);

/* ------------------------------------ one call from x (quantize + linear) --
 * y = the linear of x[M,K] (dtype xt, row-major, 16-byte aligned) in one call:
 * the activation quantizer of rsfp4_*_quantize_act_with_residue (with the
 * residue for the *_compensated calls) followed by the linear, y [M, N] stored
 * as fp32 (yt = RSFP4_F32) or bf16 (yt = RSFP4_BF16).  The sums are the ones of
 * the two calls made in turn, bit for bit.  The page fuses residue generation
 * into the quantizer, which emits the GEMM's operand layout (ResServe Section
 * 4.4), and counts an extra kernel launch as a cost (Section 4.1); this call
 * goes one step further for decode: with bf16 x, K <= 8192 and few rows to
 * quantize (MXFP4: M <= 4; NVFP4: M <= 4 plain; compensated NVFP4, whose
 * quantization is twice as long, always takes two launches), it is
 * ONE launch of the narrow linear in which every workgroup quantizes the M
 * rows itself into LDS (the same record bytes the quantizer writes, with the
 * quantizer's arithmetic) while its weight loads are in flight, and reads its
 * fragments from there; no workgroup waits for another and nothing goes
 * through HBM but x, the weights and y.  Other shapes and fp32 x run the
 * quantize and linear kernels back to back through act (with more rows the
 * quantizer, spread over M compute units, is the faster of the two).
 * act: rsfp4_packed_act_bytes(fmt, M, K, compensated) bytes of device memory,
 * 16-byte aligned, owned by the caller; holds the quantized rows after a
 * two-launch call and is left untouched by a one-launch call.  ws, ws_bytes:
 * the linear's workspace (rsfp4_workspace_bytes; NULL, 0 for none), as for the
 * linear calls.  Argument checks as for the two calls. */
/* Kernel launches such a call makes on the current device: 1 or 2 (0 for
 * arguments the calls reject). */
int rsfp4_from_x_launches(int fmt, int xt, int64_t M, int64_t N, int64_t K, int compensated);
rsfp4_status rsfp4_nvfp4_linear_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K,
                                       const void* w_packed, size_t w_packed_bytes, void* y, int yt,
                                       void* act, size_t act_bytes, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_nvfp4_linear_compensated_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K,
                                                   const void* w_packed, size_t w_packed_bytes, void* y,
                                                   int yt, void* act, size_t act_bytes, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_linear_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K,
                                       const void* w_packed, size_t w_packed_bytes, void* y, int yt,
                                       void* act, size_t act_bytes, void* ws, size_t ws_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_linear_compensated_from_x(const void* x, int xt, int64_t M, int64_t N, int64_t K,
                                                   const void* w_packed, size_t w_packed_bytes, void* y,
                                                   int yt, void* act, size_t act_bytes, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------- paper numerics: given tensor scale (NVFP4) --
 * The operator as the ResServe page's fused quantizer computes it (Appendix
 * B.2: Eq. 8 and the pack8 description; Algorithm 1), in place of the per-row
 * dynamic scale of rsfp4_nvfp4_quantize_act_with_residue:
 *   - one tensor scale alpha (fp32, device memory) for every row of x and of r
 *     (the page loads calibrated tensor scales, and the residue shares the base
 *     operand's tensor scale);
 *   - block byte S_b = E4M3_RNE((Max_b / 6) / alpha), both divisions rounded;
 *   - multiplier scale = 1 / (alpha * S_b), or 0 when alpha * S_b is 0;
 *   - element code E2M1_RNE(v * scale), sign from v;
 *   - residue r = v - e / scale (v when the scale is 0), quantized by the same
 *     steps with the same alpha.
 * Records as for rsfp4_nvfp4_quantize_act_with_residue, every record's tensor
 * scale field holding alpha; the linears above consume them unchanged (the
 * dequantized value is alpha * S_b * e).  One pass per row, x read once, no row
 * reduction. */
rsfp4_status rsfp4_nvfp4_quantize_act_alpha(const void* x, int xt, int64_t M, int64_t K,
                                            const float* alpha, int with_residue, void* act,
                                            size_t act_bytes, void* stream);

/* alpha of a whole tensor x [M, K] (dtype xt) when it is derived from the data
 * (Eq. 8: s_i = Max_i / 6, alpha = max_i s_i / 448): *alpha = ((max|x|) / 6) /
 * 448 with both divisions rounded; alpha is a device pointer to one float,
 * written by three kernels in stream order.  M * K <= 2^40. */
rsfp4_status rsfp4_nvfp4_tensor_alpha(const void* x, int xt, int64_t M, int64_t K, float* alpha,
                                      void* stream);

/* --------------------------------------- selective compensation (K-Ext) --
 * ResServe Section 5.3 ("Selective Prefill Execution", Eq. 6) and Appendix B.1
 * (Eq. 7, Algorithm 1): only k of every 8 input channels get a residue term,
 * k = 8 rho with rho in {0.125, 0.25, 0.5, 1}.  The selected residues are
 * appended to the quantized activation row and the matching weight columns to
 * W, so one plain FP4 product over K_eff = K + (K/8) k = K (1 + rho) adds the
 * base and the correction:  y = [X^ R^_S] [W^ W^_S]^T.
 *
 * Channel masks: K/8 bytes (device memory); bit j of byte g selects channel
 * 8g + j.  Each byte must have exactly k bits set (the select call makes such
 * masks); another popcount gives unspecified extension values, never an
 * out-of-bounds access.  Extension order: group after group, each group's
 * selected channels in increasing channel order.
 *
 * Flow: rsfp4_channel_abs_sum over calibration rows -> rsfp4_kext_select ->
 * masks; offline rsfp4_*_prepack_weights_kext(W, masks) -> a packed blob of
 * width K_eff; per call rsfp4_*_quantize_act_kext(x, masks) -> M records of
 * width K_eff, then rsfp4_*_linear(act, blob, M, N, K_eff) (the plain linear:
 * the sum over K_eff already holds both terms). */

/* K_eff = K + (K/8) k, or -1 unless k is 1, 2, 4 or 8, K a multiple of 32 and
 * (K/8) k a multiple of 32 (so the extension is whole blocks in both formats:
 * K % 256 == 0 for k = 1, % 128 for k = 2, % 64 for k = 4). */
int64_t rsfp4_kext_dim(int64_t K, int k);

/* Calibration score (Appendix B.1: mean absolute activation; a sum over a fixed
 * number of rows ranks channels the same way): sum[i] = (accumulate ? sum[i] :
 * 0) + |x[0, i]| + |x[1, i]| + ... + |x[T-1, i]|, added in binary64 one row
 * after another, so continuing over several batches equals one call over their
 * concatenation.  x [T, K] row-major (xt: RSFP4_F32 or RSFP4_BF16, element
 * aligned); sum: K doubles (device, 8-byte aligned).  T*K <= 2^40. */
rsfp4_status rsfp4_channel_abs_sum(const void* x, int xt, int64_t T, int64_t K, double* sum,
                                   int accumulate, void* stream);

/* Block-local selection (Eq. 7): masks[g] gets the k channels of group g with
 * the largest score; equal scores go to the lower channel index.  score: K
 * doubles (device), K % 8 == 0; masks: K/8 bytes (device).  NaN scores give
 * unspecified masks. */
rsfp4_status rsfp4_kext_select(const double* score, int64_t K, int k, uint8_t* masks, void* stream);

/* Pack [W | W_S] (W [N, K] row-major, dtype wt) into a blob of width K_eff
 * (w_packed_bytes >= rsfp4_packed_weight_bytes(fmt, N, K_eff), 256-byte
 * aligned).  Column K + p is W's column of the extension's p-th channel.  The
 * blob is quantized as one K_eff-wide tensor (Section 5.3: the selected rows
 * are appended offline and quantized in the extended block layout): NVFP4's
 * tensor scale is max|W| / 2688 (the appended columns repeat W's values), and
 * the blocks of the extension are new blocks over the gathered columns. */
rsfp4_status rsfp4_nvfp4_prepack_weights_kext(const void* W, int wt, int64_t N, int64_t K,
                                              const uint8_t* masks, int k, void* w_packed,
                                              size_t w_packed_bytes, void* stream);
rsfp4_status rsfp4_mxfp4_prepack_weights_kext(const void* W, int wt, int64_t N, int64_t K,
                                              const uint8_t* masks, int k, void* w_packed,
                                              size_t w_packed_bytes, void* stream);

/* Quantize x [M, K] into M activation records of width K_eff (act_bytes >=
 * rsfp4_packed_act_bytes(fmt, M, K_eff, 0); record layout as above with K_eff
 * in place of K).  One pass per row, x read once (Algorithm 1): row amax and
 * tensor scale s_g, base codes of all K channels, the residue r = x - deq(q(x))
 * in registers, then the selected residues quantized in their own blocks of
 * the extension -- NVFP4 with the base row's s_g (the one tensor scale of the
 * extended row), MXFP4 with the E8M0 rule.  K_eff <= 32768. */
rsfp4_status rsfp4_nvfp4_quantize_act_kext(const void* x, int xt, int64_t M, int64_t K,
                                           const uint8_t* masks, int k, void* act, size_t act_bytes,
                                           void* stream);
rsfp4_status rsfp4_mxfp4_quantize_act_kext(const void* x, int xt, int64_t M, int64_t K,
                                           const uint8_t* masks, int k, void* act, size_t act_bytes,
                                           void* stream);

/* ------------------------------------ compensated decode attention --------
 * ResAttn (ResServe Section 4.3, Eq. 3; Section 5.2 "ResAttn Execution"): one
 * decode token per sequence; the query heads of a KV head (grouped-query
 * attention, G = H_q / H_kv <= 8) are quantized to an NVFP4 base and residue,
 * both are multiplied with the cached NVFP4 keys, and their scores are added
 * before the softmax; the output is softmax(S) V^ over the cached values:
 *   S[h, t] = k_scale * sm_scale * (s_q[h] (Q^_h . K^_t) + s_r[h] (R^_h . K^_t))
 *   out[h]  = v_scale * sum_t p[h, t] V^_t / sum_t p[h, t],  p = exp(S - max S)
 * where Q^_h, R^_h, K^_t, V^_t are FP4 codes times their E4M3 block scales
 * and s_q, s_r the query rows' tensor scales.
 *
 * KV cache: pages of 32 tokens; a page holds, for each KV head in turn,
 * 36 * D bytes (NC = D / 128):
 *   [0, 16D)    K codes [32][D/2], token-major, element 2k in the low nibble;
 *   [16D, 18D)  K block scales (E4M3, 16 elements along the head dimension),
 *               D/16 bytes per row; block 8c + 2q + s (q < 4, s < 2) of row t
 *               at 16D + t D/16 + 2 NC q + 2c + s (plain block order at D = 128);
 *   [18D, 34D)  V codes in the attention kernel's operand order: row t has
 *               slot pi(t) = 8q + u, where t = 4q + u (u < 4) or
 *               t = 16 + 4q + u - 4 (u >= 4); column d = 128c + 8a + e of
 *               slot 8q + u is bits 4u..4u+3 of the 32-bit little-endian word
 *               at 18D + 2048c + 1024 (e / 4) + 16 (a + 16q) + 4 (e % 4);
 *   [34D, 36D)  V block scales: block k of row t at 34D + 32k + pi(t).
 * Token t of a sequence sits at page block_table[b][t / 32], row t % 32.  k_scale / v_scale are the cache's
 * global scales (the page's tests use 1.0): a stored value is k_scale * S_b * e.
 * D is 128 or 256. */
size_t rsfp4_kv_page_bytes(int64_t H_kv, int64_t D);

/* Quantize and write T tokens' keys and values (k, v: [T, H_kv, D], dtype xt,
 * row-major) into the cache: token t goes to slot slots[t] = page * 32 + row
 * (slots < 0 or beyond the cache are skipped).  Each 16-element block:
 * S_b = E4M3_RNE(max|x| / (6 g)), codes E2M1_RNE(x / (S_b g)), g = k_scale or
 * v_scale (> 0).  The page's timings exclude cache construction; this call is
 * how the cache is built here.  cache: device, 256-byte aligned, cache_bytes /
 * rsfp4_kv_page_bytes pages.  The slots of one call must be distinct: the V
 * codes of the 32 rows of a page share 32-bit words, and a token's nibbles are
 * replaced by two atomic steps (clear, then set), so two tokens written to one
 * slot in the same call leave the OR of their codes.  Calls that write the
 * same pages must be ordered (one stream, or synchronised); tokens of other
 * slots in the same words are left as they are. */
rsfp4_status rsfp4_kv_cache_write(const void* k, const void* v, int xt, int64_t T, int64_t H_kv, int64_t D,
                                  const int32_t* slots, float k_scale, float v_scale, void* cache,
                                  size_t cache_bytes, void* stream);

/* KV splits the preset rule picks (a power of two: at most about 8 waves per
 * compute unit over B * H_kv items, and the smallest p with p^2 B > 8 pages,
 * pages = ceil(max_seq_len / 32), i.e. about 4 sqrt(pages / B); never more than
 * the pages or 1024; ResServe Section 5.2: preset rules from batch size, KV
 * heads, sequence length and the unit count), and the workspace they need (0
 * for one split): B * H_q * splits * (D + 2) * 4 bytes. */
int rsfp4_resattn_splits(int64_t B, int64_t H_kv, int64_t max_seq_len);
size_t rsfp4_resattn_workspace_bytes(int64_t B, int64_t H_q, int64_t D, int splits);

/* Decode attention of B sequences.
 *   q_act:       query records from rsfp4_nvfp4_quantize_act_with_residue over
 *                q viewed as [B * H_q, D] rows (with_residue = compensated);
 *   compensated: 0 = scores from the base only (plain NVFP4 query);
 *   block_table: [B, max_pages] int32 page indices (device); seq_lens: [B]
 *                int32 (device), each <= max_seq_len <= 32 * max_pages (tokens
 *                beyond max_seq_len are not read);
 *   sm_scale:    usually 1 / sqrt(D);
 *   splits:      KV splits (<= 0: the preset rule); with more than one, the
 *                workspace ws (device, 16-byte aligned, at least
 *                rsfp4_resattn_workspace_bytes) holds the partial outputs
 *                and a second kernel combines them;
 *   out:         [B, H_q, D], fp32 or (out_bf16) bf16, fully overwritten
 *                (a sequence of length 0 gives zeros).
 * Page indices outside the cache read as zeros. */
rsfp4_status rsfp4_resattn_decode(const void* q_act, size_t q_act_bytes, int compensated, const void* cache,
                                  size_t cache_bytes, const int32_t* block_table, int64_t max_pages,
                                  const int32_t* seq_lens, int64_t max_seq_len, int64_t B, int64_t H_q,
                                  int64_t H_kv, int64_t D, float k_scale, float v_scale, float sm_scale,
                                  int splits, void* out, int out_bf16, void* ws, size_t ws_bytes,
                                  void* stream);

/* ------------------------------------------------------- test / debug ----
 * Rewrite a packed blob in canonical row-major form: codes[N, K/2] (low nibble
 * = even K index), scales[N, K/blk], and (NVFP4) the tensor scale to *s_g
 * (a device pointer to one float; may be NULL for MXFP4).  Enqueued on stream. */
rsfp4_status rsfp4_unpack_weights_canonical(const void* w_packed, size_t w_packed_bytes, int fmt,
                                            int64_t N, int64_t K, uint8_t* codes, uint8_t* scales,
                                            float* s_g, void* stream);

/* Test/measurement: read `bytes` bytes at src (device memory, 16-byte aligned)
 * once, at the rate a kernel that only reads achieves (one workgroup of 8
 * waves per compute unit, each sweeping a contiguous chunk with non-temporal
 * 16-byte loads, two per wave in flight).  Timed at the byte count of a
 * linear's weight stream it gives the measured streaming-read ceiling that
 * the linear's HBM rate is compared with, beside the nominal peak.  The
 * kernel folds every 32-bit word of the buffer with xor and xors the result
 * into *sink (4 bytes of device memory, 4-byte aligned; atomically, one
 * atomic per workgroup), so that the loads cannot be dropped and a caller
 * that zeroes sink first reads back the xor of the whole buffer.  bytes: a
 * multiple of 16 (else RSFP4_ERR_SHAPE), at
 * most 1 GiB per compute unit (else RSFP4_ERR_UNSUPPORTED).  Enqueues one
 * kernel on `stream`. */
rsfp4_status rsfp4_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/* Test/debug: check a packed weight blob's 256-byte header against the rules
 * of the layout above (magic, ABI version, format, N and K in range, tensor
 * scale finite and non-negative for NVFP4 and zero for MXFP4, w_packed_bytes
 * at least the size query for the header's format, N, K) and report the
 * header's format, N and K (each output may be NULL).  Copies the header to
 * the host on `stream` and SYNCHRONIZES that stream.  A bad header returns
 * RSFP4_ERR_FORMAT, a short buffer RSFP4_ERR_BUFFER_TOO_SMALL. */
rsfp4_status rsfp4_validate_packed(const void* w_packed, size_t w_packed_bytes, int* fmt, int64_t* N, int64_t* K,
                                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RSFP4_H */
