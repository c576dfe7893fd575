// nvfp4_probe.hip -- measurement aids, not part of the GEMM path: the two
// floors that bound the decode-sized calls on this GPU, the per-call cost of
// a kernel that does nothing, and the latency of one dependent load from L2,
// from the last-level cache or from HBM (a single work-item walking a
// random cycle through a buffer of chosen size); and the two measured peaks
// the GEMM kernels are compared with besides the datasheet figures, the rate
// of fp16 MFMA work and of streaming reads from HBM on this GPU.
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

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

// MFMA rate: every wave runs `iters` rounds of 8 independent
// v_mfma_f32_32x32x16_f16 (enough in flight to keep the matrix unit busy),
// on operands built from the lane index (ordinary values in [-1, 1), since
// the clock the chip sustains depends on the data), then writes the sum of
// its accumulators, so no MFMA can be dropped.  4 waves per workgroup.
__global__ void __launch_bounds__(256) probe_mfma_kernel(int iters, float* out) {
    const int lane = threadIdx.x & 63;
    h8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)((float)((lane * 37 + i * 11) & 127) / 64.0f - 1.0f);
        b[i] = (_Float16)((float)((lane * 53 + i * 29 + 7) & 127) / 64.0f - 1.0f);
    }
    f16v acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f16v{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming read: the grid reads `chunks` 16-byte chunks of src once, each
// work-item four chunks per round (all four loads in flight before the
// first is used), and folds them into one word that is stored only if it
// equals `never` (so the loads cannot be dropped and nothing is written in
// practice).  Chunks are dealt round-robin over the whole grid, so every
// load instruction of a wave reads 1 KB of consecutive bytes.
__global__ void __launch_bounds__(256) probe_read_kernel(const uint4* __restrict__ src,
                                                         int64_t chunks, uint32_t never,
                                                         uint32_t* out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < chunks; i += 4 * stride) {
        const uint4 v0 = src[i], v1 = src[i + stride], v2 = src[i + 2 * stride], v3 = src[i + 3 * stride];
        acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
        acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
    }
    for (; i < chunks; i += stride) {
        const uint4 v = src[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never) out[0] = acc;
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

int nvfp4_probe_mfma(int64_t blocks, int64_t iters, float* out, void* stream) {
    if (!out || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > INT32_MAX)
        return NVFP4_ERR_INVALID_VALUE;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), (int)iters, out);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_probe_read(const void* src, int64_t bytes, int64_t blocks, uint32_t* out,
                     void* stream) {
    if (!src || !out || bytes < 16 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20) ||
        (reinterpret_cast<uintptr_t>(src) & 15u))
        return NVFP4_ERR_INVALID_VALUE;
    hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16,
                       0x9E3779B9u, out);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
