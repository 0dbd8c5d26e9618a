// stream_read.hip -- a plain streaming read of a device buffer: the rate the
// memory system delivers to a kernel that does nothing but read, measured at
// the byte count of a weight stream, as the ceiling the linear's HBM rate is
// compared against (beside the nominal peak).
//
// Shape (from a sweep of waves per workgroup, loads in flight per wave,
// workgroups per CU, chunk order and cache policy at 9.4-132 MB): one
// workgroup of 8 waves per CU, each workgroup sweeping a contiguous chunk of
// the buffer with its waves interleaved 2 KB apart, two 1 KB loads per wave in
// flight at a time (double-buffered), non-temporal loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_frag.h"
#include "kernels.h"

namespace rsfp4 {

namespace {

constexpr int kReadWaves = 8;
constexpr int kReadLoads = 2;                       // 1 KB wave loads per wave and turn
constexpr uint32_t kTurn = kReadWaves * kReadLoads * 1024;   // bytes a workgroup reads per turn

__global__ __launch_bounds__(64 * kReadWaves) void stream_read_kernel(const uint8_t* src, int64_t bytes,
                                                                      int64_t chunk, uint32_t* sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    if (lo >= bytes) return;
    const int64_t n = bytes - lo < chunk ? bytes - lo : chunk;      // this workgroup's bytes (< 2^32)
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc((void*)(src + lo), (short)0, (int)n, kRsrcWord3);
    const uint32_t first = (uint32_t)wave * kReadLoads * 1024u + 16u * lane;
    const uint32_t turns = (uint32_t)((n + kTurn - 1) / kTurn);
    u32x4 a[kReadLoads], b[kReadLoads];
    uint32_t acc = 0;
    // out-of-range offsets (the chunk's tail) read zeros without a memory access
    auto load = [&](u32x4 (&v)[kReadLoads], uint32_t t) {
#pragma unroll
        for (int l = 0; l < kReadLoads; ++l)
            v[l] = __builtin_amdgcn_raw_buffer_load_b128(r, first + t * kTurn + l * 1024u, 0, kStreamPolicy);
    };
    auto fold = [&](const u32x4 (&v)[kReadLoads]) {
#pragma unroll
        for (int l = 0; l < kReadLoads; ++l) acc ^= v[l][0] ^ v[l][1] ^ v[l][2] ^ v[l][3];
    };
    load(a, 0);
    for (uint32_t t = 0; t < turns; t += 2) {
        load(b, t + 1);
        fold(a);
        load(a, t + 2);
        fold(b);
    }
    // the xor of every word the workgroup read goes into *sink with one
    // atomic: the loads stay live and a caller can check what was read
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
    __shared__ uint32_t part[kReadWaves];
    if (lane == 0) part[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t v = 0;
#pragma unroll
        for (int w = 0; w < kReadWaves; ++w) v ^= part[w];
        atomicXor(sink, v);
    }
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int num_cus, hipStream_t s) {
    if (bytes <= 0) return hipSuccess;
    int64_t chunk = (bytes + num_cus - 1) / num_cus;
    chunk = (chunk + kTurn - 1) / kTurn * kTurn;
    if (chunk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t grid = (bytes + chunk - 1) / chunk;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(64 * kReadWaves), 0, s,
                       static_cast<const uint8_t*>(src), bytes, chunk, sink);
    return hipGetLastError();
}

}  // namespace rsfp4
