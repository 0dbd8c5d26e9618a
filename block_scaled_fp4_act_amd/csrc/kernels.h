// kernels.h -- internal launchers of the gfx950 kernels (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsfp4 {

// The per-row quantizer; with few rows (M x parts within num_cus) a row is
// shared by up to 8 workgroups (num_cus = 0: one workgroup per row).
hipError_t launch_quantize_act(int fmt, int xt_bf16, const void* x, int M, int64_t K, int with_res,
                               void* act, int num_cus, hipStream_t s);

hipError_t launch_prepack(int fmt, int wt_bf16, const void* W, int64_t N, int64_t K, void* blob,
                          hipStream_t s);

// Compensated decode attention (ResAttn) over the paged NVFP4 KV cache.
int64_t kv_page_bytes(int64_t H_kv, int64_t D);
hipError_t launch_kv_write(int xt_bf16, const void* k, const void* v, const int32_t* slots, int64_t T, int H_kv,
                           int D, float k_scale, float v_scale, void* cache, int64_t num_pages, hipStream_t s);
int attn_auto_splits(int64_t B, int64_t H_kv, int64_t max_seq_len, int num_cus);
hipError_t launch_resattn(const void* q_act, int64_t q_row_bytes, int comp, const void* cache, int64_t num_pages,
                          const int32_t* block_table, int64_t max_pages, const int32_t* seq_lens, int B, int H_q,
                          int H_kv, int D, float k_scale, float v_scale, float sm_scale, int splits,
                          int64_t max_seq_len, void* out, int out_bf16, float* ws, hipStream_t s);

// Selective compensation (K-Ext): extended quantizer, [W | W_S] prepack and the
// calibration kernels.
hipError_t launch_quantize_act_kext(int fmt, int xt_bf16, const void* x, int M, int64_t K,
                                    const uint8_t* masks, int k, void* act, hipStream_t s);
hipError_t launch_prepack_kext(int fmt, int wt_bf16, const void* W, int64_t N, int64_t Kb,
                               const uint8_t* masks, int k, void* blob, hipStream_t s);
hipError_t launch_channel_abs_sum(int xt_bf16, const void* x, int64_t T, int64_t K, double* sum,
                                  int accumulate, hipStream_t s);
hipError_t launch_kext_select(const double* score, int64_t K, int k, uint8_t* masks, hipStream_t s);

hipError_t launch_unpack(int fmt, const void* blob, int64_t N, int64_t K, uint8_t* codes,
                         uint8_t* scales, float* s_g, hipStream_t s);

// Launch shape of the narrow-M linear: rt row tiles of 16, maxs steps per wave,
// kw waves per workgroup along K, grid workgroups (grid-stride over channel groups).
struct GemmPlan {
    int rt = 1;
    int maxs = 1;
    int kw = 1;
    int64_t grid = 1;
    int ngl = 1;       // groups reduced together (partial sums held in LDS)
    int ks = 1;        // K slices split across workgroups (1: each workgroup covers the launch's K)
    int ss = 0;        // steps per slice (ks > 1: kw * maxs)
};

// Plan for a launch over `steps` K steps of 128 (at most 128 steps).  With
// split_ok the plan may split K across workgroups (ks > 1), which needs a
// workspace of split_ws_bytes(plan, ...) bytes.
GemmPlan plan_gemm_small(int64_t M, int64_t N, int64_t steps, bool comp, int num_cus, bool split_ok = false);

// Workspace of a split plan: kSplitGroups zero-initialised int counters (one
// per channel group; a fixed area, so calls of any shape can share one
// workspace: each call leaves the counters it used at zero), then one
// partial-sum record per group and slice.  Plans split only N of at most
// kSplitGroups groups.
constexpr int64_t kSplitGroups = 4096;
constexpr int64_t kSplitCounterBytes = kSplitGroups * 4;
int64_t split_ws_bytes(const GemmPlan& pl, bool comp, int64_t N);

// Streaming read of bytes bytes at src (one workgroup of 8 waves per CU), the
// reference rate for the weight stream; the xor of all its 32-bit words is
// xor-ed into *sink.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int num_cus, hipStream_t s);

// The library's per-device scratch (scratch.hip): its size, and its device
// address on the current device (taken on the first call per device, which
// also clears the counter area on stream s).
int64_t scratch_bytes();
hipError_t scratch_ptr(hipStream_t s, void** out);

// One launch over steps [s_lo, s_hi) of K (s_lo a multiple of 8); accum adds
// the result to y (the second launch of a K longer than one launch covers).
// ws: the split plan's workspace (unused when pl.ks == 1); its counters must be
// zero on entry and are zero again when the launch completes.
hipError_t launch_gemm_small(int fmt, const GemmPlan& pl, bool comp, const void* act,
                             int64_t row_bytes, const void* blob, int M, int64_t N, int64_t K,
                             void* y, bool out_bf16, int s_lo, int s_hi, bool accum, void* ws, hipStream_t s);

// Grouped (mixture of experts) narrow linear, one launch: expert e multiplies
// rows offsets[e] .. offsets[e+1] (at most max_rows) of an act buffer of M_total
// rows by the e-th of E stacked blobs (blob_stride bytes apart) into the same
// rows of y (fp32).  Plan with plan_gemm_small(max_rows, N, steps, comp,
// num_cus / E) so the E x grid workgroups fit the device.
hipError_t launch_gemm_grouped(int fmt, const GemmPlan& pl, bool comp, const void* act, int64_t row_bytes,
                               int M_total, const void* blobs, int64_t blob_stride, int E, const int32_t* offsets,
                               int max_rows, int64_t N, int64_t K, float* y, hipStream_t s);

// Narrow linear that quantizes its own activation rows (bf16 x[M, K]) in every
// workgroup, into LDS records (the quantize kernel's bytes), in one launch.
struct InqPlan {
    bool ok = false;   // the shape fits this kernel
    GemmPlan pl;
    int qrow = 64;     // threads per quantized row
    int ncq = 2;       // chunks of 8 elements per thread
};
InqPlan plan_gemm_inq(int fmt, int64_t M, int64_t N, int64_t K, bool comp, int num_cus);
hipError_t launch_gemm_inq(int fmt, const InqPlan& q, bool comp, const void* x, const void* blob, int M, int64_t N,
                           int64_t K, void* y, bool out_bf16, hipStream_t s);

// Wide-operand linear (any number of activation rows): 2-D tiles of 128 rows x
// 128 channels per workgroup, each wave walking all of K.
hipError_t launch_gemm_tile(int fmt, bool comp, const void* act, int64_t row_bytes, const void* blob,
                            int M, int64_t N, int64_t K, void* y, bool out_bf16, hipStream_t s);

// Wide-operand MXFP4 linear over LDS-DMA streamed operands: the activation
// records rewritten into the packed-weight layout (groups of 16 stacked rows,
// base and residue rows interleaved; act_tile_bytes bytes), then the tiled
// product of the two (gemm_tile_dma.hip).
int64_t act_tile_bytes(int fmt, int64_t B, int64_t K);
hipError_t launch_act_tile(int fmt, bool comp, const void* act, int64_t row_bytes, int M, int64_t K, void* out,
                           hipStream_t s);
hipError_t launch_gemm_tile_dma(bool comp, const void* act_tiled, const void* blob, int M, int64_t N, int64_t K,
                                void* y, bool out_bf16, int num_cus, hipStream_t s);
// NVFP4: the activations rewritten as exact f16 MFMA fragments (4 KB per 16
// rows and step), streamed into LDS by DMA; weights from a register ring.
// With few tiles K is split into ks slices (nv_tile_split; at most
// kMaxTileSplit) whose folded partial sums (nv_split_bytes at part) are added in
// slice order by the last slice to arrive at its counter (cnt: the zeroed
// counter area of kSplitGroups ints, left zero).
constexpr int kMaxTileSplit = 8;
int nv_tile_split(int64_t B, int64_t N, int64_t K, int num_cus);
int64_t nv_split_bytes(int64_t B, int64_t N, int ks, bool comp);
hipError_t launch_gemm_tile_dma_nv(bool comp, const void* act_tiled, const void* act, int64_t row_bytes,
                                   const void* blob, int M, int64_t N, int64_t K, void* y, bool out_bf16,
                                   int ks, int* cnt, float* part, hipStream_t s);

// Paper-numerics NVFP4 quantizer (tensor scale alpha from device memory, shared
// by x and r; multiplier-scale codes and residue) and the alpha of a tensor.
hipError_t launch_quantize_act_alpha(int xt_bf16, const void* x, int M, int64_t K, const float* alpha,
                                     int with_res, void* act, hipStream_t s);
hipError_t launch_tensor_alpha(int xt_bf16, const void* x, int64_t n, float* alpha, hipStream_t s);

}  // namespace rsfp4
