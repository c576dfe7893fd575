// nvfp4_host.h -- host-side pieces shared by the eager entry points and the
// recorded sequences (not part of the public ABI): a validated and planned
// launch ("job"), the device check, and the launch of a job.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nvfp4_internal.h"
#include "nvfp4_plan.h"

namespace nvfp4 {

enum JobKind {
    JOB_GEMM = 0,
    JOB_GROUPED = 1,
    JOB_QUANTIZE = 2,
    JOB_GROUPED_TILE = 3,
    JOB_GEMV_QUANT = 4,
    JOB_GROUPED_WSPLIT = 5
};

struct Job {
    int kind = JOB_GEMM;
    Plan plan{};                 // JOB_GEMM (JOB_GROUPED_TILE: plan.cfg)
    GemmArgs gemm{};             // JOB_GEMM, JOB_GROUPED_TILE (workspace pointers set at launch)
    size_t floats = 0;           // split-K partial floats the job needs (tile, wsplit)
    size_t flagged = 0;          // flagged 64-bit partial words the job needs (skinny)
    size_t counters = 0;         // split-K arrival counters the job needs
    GroupedArgs grouped{};       // JOB_GROUPED, JOB_GROUPED_WSPLIT
    QuantArgs quant{};           // JOB_QUANTIZE
    GemvQuantArgs gemvq{};       // JOB_GEMV_QUANT
    bool empty = false;          // nothing to launch (a grouped GEMM with no rows)
};

// Argument checks and planning, host-only (no device call).  Return an
// NVFP4_* status; on NVFP4_OK the job is ready to launch.
int prepare_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
                 const void* b_scales, float alpha, void* out, int64_t M, int64_t N, int64_t K,
                 int path, int tile, int split_k, Job* job);
int prepare_grouped(const void* a_packed, const void* a_scales, const void* b_packed,
                    const void* b_scales, const int32_t* row_offsets, int64_t groups, float alpha,
                    void* out, int64_t M, int64_t N, int64_t K, int path, Job* job);
int prepare_quantize(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld,
                     void* packed_codes, void* packed_scales, Job* job);
int prepare_gemm_quantized(const void* x, int x_type, int64_t ldx, const void* b_packed,
                           const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                           int64_t K, Job* job);

// The current device, checked to be a gfx950 GPU (status).
int current_device(int* device);

// The split-K workspace of a launch.  Counters and flagged words are zero
// between calls (every kernel that uses them leaves them so); the FP32
// partials need no initial value.
struct WorkspacePtrs {
    float* partials = nullptr;
    uint64_t* flagged = nullptr;
    uint32_t* counters = nullptr;
};

// Enqueues a prepared job on `stream`, with the split-K workspace given
// (null pointers when the job needs none).
hipError_t launch_job(const Job& job, int device, const WorkspacePtrs& ws, hipStream_t stream);

}  // namespace nvfp4
