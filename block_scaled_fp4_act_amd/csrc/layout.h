// layout.h -- byte layouts shared by the host API and the gfx950 kernels.
//
// Activation buffer: one fixed-stride record per quantized row, base rows then
// residue rows (the stacked operand [X^; R^] of Eq. 2 on the ResServe page,
// Section 4.3).  Packed weights: a header, then groups of 16 output channels,
// each a sequence of 128-element K steps whose 1 KB of codes is exactly one
// 64-lane, 16-bytes-per-lane load, followed by that step's block scales.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define RSFP4_HD __host__ __device__

namespace rsfp4 {

constexpr int kNV = 0;  // NVFP4
constexpr int kMX = 1;  // MXFP4

RSFP4_HD constexpr int block_elems(int fmt) { return fmt == kNV ? 16 : 32; }

// ---- activation records ----
constexpr int64_t kActHead = 16;  // fp32 tensor scale + pad; codes start 16-aligned

RSFP4_HD inline int64_t act_row_bytes(int fmt, int64_t K) {
    int64_t b = kActHead + K / 2 + K / block_elems(fmt);
    return (b + 15) / 16 * 16;
}

// ---- packed weights ----
constexpr int64_t kWHeader = 256;
constexpr int64_t kStepK = 128;             // K elements per step
constexpr int64_t kStepCodes = 1024;        // 16 channels x 128 K / 2
constexpr int64_t kGroupN = 16;             // output channels per group

RSFP4_HD constexpr int64_t step_scale_bytes(int fmt) { return fmt == kNV ? 128 : 64; }
RSFP4_HD constexpr int64_t step_bytes(int fmt) { return kStepCodes + step_scale_bytes(fmt); }

RSFP4_HD inline int64_t num_steps(int64_t K) { return (K + kStepK - 1) / kStepK; }
RSFP4_HD inline int64_t num_groups(int64_t N) { return (N + kGroupN - 1) / kGroupN; }
RSFP4_HD inline int64_t group_bytes(int fmt, int64_t K) { return num_steps(K) * step_bytes(fmt); }
RSFP4_HD inline int64_t packed_weight_bytes(int fmt, int64_t N, int64_t K) {
    return kWHeader + num_groups(N) * group_bytes(fmt, K);
}

constexpr uint32_t kMagic = 0x34465352u;  // "RSF4"

struct WHeader {            // first bytes of the 256-byte header (device memory)
    uint32_t magic;
    uint32_t abi_version;
    uint32_t fmt;
    uint32_t amax_bits;     // max|W| as binary32 bits (NVFP4), reduced by atomicMax
    int64_t N;
    int64_t K;
    float s_g;              // NVFP4 tensor scale amax / 2688; 0 for MXFP4
    uint32_t pad[7];
};
static_assert(sizeof(WHeader) <= kWHeader, "header too large");

}  // namespace rsfp4
