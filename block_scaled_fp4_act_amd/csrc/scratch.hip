// scratch.hip -- the library's own device workspace for callers that cannot
// allocate (code under stream capture, serving loops, harnesses that forbid
// device allocation): a file-scope device array, one per GPU, used in place
// of a caller's workspace by the no-allocation linear entry point.
//
// In host code `scratch` names a host-side stand-in of the symbol, not device
// memory; the device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept in g_ptr[device].  Only that
// address is ever handed to a kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "kernels.h"

namespace rsfp4 {

namespace {

// The split linear's counters (kSplitCounterBytes, zero between calls) and
// partial sums: enough for every plan plan_gemm_small splits (at most
// kSplitGroups groups x 4 slices x 1 KB: two row tiles, K = 16384; one row
// tile takes at most 2 slices of 512 bytes per group, or 4 of 256 groups).
constexpr int64_t kScratchBytes = kSplitCounterBytes + kSplitGroups * 4 * 1024;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDev = 64;
std::once_flag g_once[kMaxDev];
void* g_ptr[kMaxDev];
hipError_t g_err[kMaxDev];

__global__ void clear_words(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

}  // namespace

int64_t scratch_bytes() { return kScratchBytes; }

hipError_t scratch_ptr(hipStream_t s, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::call_once(g_once[dev], [dev, s] {
        void* p = nullptr;
        hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (r == hipSuccess) {
            // the counters must start at zero; every call leaves them zero
            hipLaunchKernelGGL(clear_words, dim3(16), dim3(256), 0, s, static_cast<uint32_t*>(p),
                               kSplitCounterBytes / 4);
            r = hipGetLastError();
        }
        g_ptr[dev] = r == hipSuccess ? p : nullptr;
        g_err[dev] = r;
    });
    if (g_err[dev] != hipSuccess) return g_err[dev];
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace rsfp4
