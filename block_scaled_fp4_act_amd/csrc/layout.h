// layout.h -- byte layouts shared by the host API and the gfx950 kernels.
//
// Activation buffer: one fixed-stride record per quantized row, base rows then
// residue rows (the stacked operand [X^; R^] of Eq. 2 on the ResServe page,
// Section 4.3).  Packed weights: a header, then groups of 16 output channels,
// each a sequence of 128-element K steps whose 1 KB of codes is exactly one
// 64-lane, 16-bytes-per-lane load; block scales follow every 4 steps.
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
// A group (16 output channels) is a run of "quads" of 4 K-steps of 128
// elements (the last quad padded with zero codes).  A quad holds its steps' codes (1 KB per step: lane l = 16g + i of
// a 64-lane load owns channel i, elements 32g..32g+31 of the step, 16 bytes)
// followed by the quad's block scales laid out per lane: lane l's scale bytes
// for the quad's 4 steps are adjacent (NVFP4: 2 bytes per step = E4M3 of blocks
// 2g, 2g+1; MXFP4: 1 byte per step = the E8M0 of block g), so a wave reads the
// scales of all its steps in one load.
constexpr int64_t kWHeader = 256;
constexpr int64_t kStepK = 128;             // K elements per step
constexpr int64_t kStepCodes = 1024;        // 16 channels x 128 K / 2
constexpr int64_t kGroupN = 16;             // output channels per group
constexpr int64_t kQuadSteps = 4;

RSFP4_HD constexpr int64_t scale_bytes_per_step_lane(int fmt) { return fmt == kNV ? 2 : 1; }
RSFP4_HD constexpr int64_t quad_scale_bytes(int fmt) { return 64 * kQuadSteps * scale_bytes_per_step_lane(fmt); }
RSFP4_HD constexpr int64_t quad_bytes(int fmt) { return kQuadSteps * kStepCodes + quad_scale_bytes(fmt); }

RSFP4_HD inline int64_t num_steps(int64_t K) { return (K + kStepK - 1) / kStepK; }
RSFP4_HD inline int64_t num_groups(int64_t N) { return (N + kGroupN - 1) / kGroupN; }
// Groups hold whole quads: the codes of steps past the last one are zero.
RSFP4_HD inline int64_t num_quads(int64_t K) { return (num_steps(K) + kQuadSteps - 1) / kQuadSteps; }
RSFP4_HD inline int64_t group_bytes(int fmt, int64_t K) { return num_quads(K) * quad_bytes(fmt); }
// Offset inside a group of step s's codes, and of the scale area of the quad
// holding step s (lane l's entry starts l * 4 * scale_bytes later).
RSFP4_HD inline int64_t step_code_offset(int fmt, int64_t s) {
    return (s / kQuadSteps) * quad_bytes(fmt) + (s % kQuadSteps) * kStepCodes;
}
RSFP4_HD inline int64_t quad_scale_offset(int fmt, int64_t s) {
    return (s / kQuadSteps) * quad_bytes(fmt) + kQuadSteps * kStepCodes;
}
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
