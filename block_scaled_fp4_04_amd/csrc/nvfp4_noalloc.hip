// nvfp4_noalloc.hip -- the GEMM entry point that allocates nothing
// (nvfp4_gemm_noalloc, include/nvfp4.h), for callers that cannot allocate
// device memory: code under graph capture, tight serving loops, harnesses
// that forbid it.
//
// The split-K workspace (arrival counters, then flagged partial words, then
// FP32 partial tiles) is a file-scope device array of fixed size instead of
// a library allocation.
// Each device holds its own copy of the array, at its own address, for the
// life of the process.  In host code the array's name stands for a host-side
// shadow, not for device memory, so the host never passes it to a kernel:
// the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and that address is what the kernels receive.
//
// The array is zero when the code object is loaded, and every kernel that
// uses a counter or a flagged word leaves it at zero again when it finishes
// (the last arrival resets its counter and clears the words it read; a
// two-way hand-off that gives up takes its increments back), so every call
// finds them at zero without a fill.
#include <hip/hip_runtime.h>

#include <mutex>

#include "nvfp4.h"
#include "nvfp4_host.h"

using namespace nvfp4;

namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static_assert(kScratchBytes == NVFP4_NOALLOC_SCRATCH_BYTES &&
                  kScratchCounters == NVFP4_NOALLOC_MAX_COUNTERS,
              "scratch size as declared in nvfp4.h");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

// Device address of this device's scratch array (looked up on first use).
int scratch_of(int device, uint8_t** ptr) {
    if (device < 0 || device >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int current = 0;
        if (hipGetDevice(&current) != hipSuccess) return NVFP4_ERR_HIP;
        if (current != device && hipSetDevice(device) != hipSuccess) return NVFP4_ERR_HIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (current != device) (void)hipSetDevice(current);
        if (e != hipSuccess || !p) return NVFP4_ERR_HIP;
        g_scratch_ptr[device] = static_cast<uint8_t*>(p);
    }
    *ptr = g_scratch_ptr[device];
    return NVFP4_OK;
}

// Whether the array holds what a job's plan needs.
bool fits(const Job& job) {
    return job.counters <= kScratchCounters && job.flagged <= kScratchFlaggedWords &&
           job.floats <= kScratchPartialFloats;
}

}  // namespace

namespace nvfp4 {

int noalloc_setup(int device) {
    uint8_t* p = nullptr;
    return scratch_of(device, &p);
}

}  // namespace nvfp4

extern "C" {

int nvfp4_noalloc_scratch_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
    if (!bytes) return NVFP4_ERR_INVALID_VALUE;
    // alignment-valid stand-in pointers: only the plan is wanted here
    const void* p = reinterpret_cast<const void*>((uintptr_t)256);
    Job job;
    const int st = prepare_gemm(p, p, p, p, 1.0f, const_cast<void*>(p), M, N, K, NVFP4_PATH_AUTO,
                                0, 0, &job);
    if (st != NVFP4_OK) return st;
    *bytes = job.counters * sizeof(uint32_t) + job.flagged * sizeof(uint64_t) +
             job.floats * sizeof(float);
    return fits(job) ? NVFP4_OK : NVFP4_ERR_SCRATCH;
}

int nvfp4_gemm_noalloc(const void* a_packed, const void* a_scales, const void* b_packed,
                       const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                       int64_t K, void* stream) {
    Job job;
    int st = prepare_gemm(a_packed, a_scales, b_packed, b_scales, alpha, out, M, N, K,
                          NVFP4_PATH_AUTO, 0, 0, &job);
    if (st != NVFP4_OK) return st;
    if (!fits(job)) return NVFP4_ERR_SCRATCH;
    int device = 0;
    st = current_device(&device);
    if (st != NVFP4_OK) return st;
    WorkspacePtrs ws;
    if (job.floats || job.flagged || job.counters) {
        uint8_t* base = nullptr;
        st = scratch_of(device, &base);
        if (st != NVFP4_OK) return st;
        ws.counters = reinterpret_cast<uint32_t*>(base);
        ws.flagged = reinterpret_cast<uint64_t*>(base + kScratchCounters * sizeof(uint32_t));
        ws.partials = reinterpret_cast<float*>(base + kScratchCounters * sizeof(uint32_t) +
                                               kScratchFlaggedWords * sizeof(uint64_t));
    }
    const hipError_t e = launch_job(job, device, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // extern "C"
