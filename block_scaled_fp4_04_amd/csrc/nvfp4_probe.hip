// nvfp4_probe.hip -- measurement aids, not part of the GEMM path: the two
// floors that bound the decode-sized calls on this GPU, the per-call cost of
// a kernel that does nothing, and the latency of one dependent load from L2,
// from the last-level cache or from HBM (a single work-item walking a
// random cycle through a buffer of chosen size).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace {

__global__ void probe_empty_kernel() {}

// One work-item follows next[] from index 0; every load depends on the one
// before.  n is a power of two and the index is masked by n - 1, so no
// content of next[] can take a load outside the array.  The loop always
// ends after `steps` loads.
__global__ void probe_chase_kernel(const uint32_t* next, uint32_t mask, int64_t steps,
                                   uint32_t* out) {
    uint32_t i = 0;
    for (int64_t s = 0; s < steps; ++s) i = next[i] & mask;
    *out = i;
}

}  // namespace

extern "C" {

int nvfp4_probe_empty(int64_t blocks, int64_t threads, void* stream) {
    if (blocks < 1 || blocks > INT32_MAX || threads < 1 || threads > 1024)
        return NVFP4_ERR_INVALID_VALUE;
    hipLaunchKernelGGL(probe_empty_kernel, dim3((unsigned)blocks), dim3((unsigned)threads), 0,
                       static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_probe_chase(const uint32_t* next, int64_t n, int64_t steps, uint32_t* out,
                      void* stream) {
    if (!next || !out || n < 1 || n > ((int64_t)1 << 32) || (n & (n - 1)) != 0 || steps < 0)
        return NVFP4_ERR_INVALID_VALUE;
    hipLaunchKernelGGL(probe_chase_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream),
                       next, (uint32_t)(n - 1), steps, out);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
