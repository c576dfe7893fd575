// nvfp4_sequence.cpp -- recorded sequences of NVFP4 calls, replayed with one
// HIP graph launch (include/nvfp4.h, "Recorded sequences").
//
// Decode steps run the same few small GEMMs for every token, each worth a
// few microseconds of device time; launching them one by one costs about as
// much again ("Peeling the Kernel Onion", section "Knowledge Created and Its
// Impact": graphs to cut launch overhead for small GEMMs).  A sequence keeps
// the validated, planned calls; finalize captures them, in order, on a
// private stream into a graph that owns nothing but kernel nodes (the
// workspace is zeroed once with a synchronous fill before the capture; the
// kernels leave counters and ready flags clear again, so no memset node is
// ever recorded), and launch replays that graph.
#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "nvfp4.h"
#include "nvfp4_host.h"

using namespace nvfp4;

struct nvfp4_sequence {
    std::vector<Job> jobs;
    bool finalized = false;
    int device = -1;
    WorkspacePtrs ws;   // the sequence's own split-K workspace
    hipGraphExec_t exec = nullptr;
};

namespace {

int add_job(nvfp4_sequence* seq, int status, const Job& job) {
    if (status != NVFP4_OK) return status;
    seq->jobs.push_back(job);
    return NVFP4_OK;
}

void release(nvfp4_sequence* seq) {
    if (seq->exec) (void)hipGraphExecDestroy(seq->exec);
    if (seq->ws.partials) (void)hipFree(seq->ws.partials);
    if (seq->ws.flagged) (void)hipFree(seq->ws.flagged);
    if (seq->ws.counters) (void)hipFree(seq->ws.counters);
    seq->exec = nullptr;
    seq->ws = WorkspacePtrs{};
}

// Captures the jobs on a private stream and instantiates the graph.
int capture(nvfp4_sequence* seq) {
    hipStream_t cs = nullptr;
    if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return NVFP4_ERR_HIP;
    int st = NVFP4_OK;
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
        st = NVFP4_ERR_HIP;
    } else {
        for (const Job& job : seq->jobs) {
            if (launch_job(job, seq->device, seq->ws, cs) != hipSuccess) {
                st = NVFP4_ERR_HIP;
                break;
            }
        }
        // always end the capture, so the stream can be destroyed
        if (hipStreamEndCapture(cs, &graph) != hipSuccess) st = NVFP4_ERR_HIP;
    }
    if (st == NVFP4_OK && hipGraphInstantiate(&seq->exec, graph, nullptr, nullptr, 0) != hipSuccess) {
        seq->exec = nullptr;
        st = NVFP4_ERR_HIP;
    }
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(cs);
    return st;
}

}  // namespace

extern "C" {

int nvfp4_sequence_create(nvfp4_sequence_t* seq) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    *seq = new (std::nothrow) nvfp4_sequence();
    return *seq ? NVFP4_OK : NVFP4_ERR_ALLOC;
}

int nvfp4_sequence_add_gemm(nvfp4_sequence_t seq, const void* a_packed, const void* a_scales,
                            const void* b_packed, const void* b_scales, float alpha, void* out,
                            int64_t M, int64_t N, int64_t K) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (seq->finalized) return NVFP4_ERR_STATE;
    Job job;
    const int st = prepare_gemm(a_packed, a_scales, b_packed, b_scales, alpha, out, M, N, K,
                                NVFP4_PATH_AUTO, 0, 0, &job);
    return add_job(seq, st, job);
}

int nvfp4_sequence_add_grouped_gemm(nvfp4_sequence_t seq, const void* a_packed,
                                    const void* a_scales, const void* b_packed,
                                    const void* b_scales, const int32_t* row_offsets,
                                    int64_t groups, float alpha, void* out, int64_t M, int64_t N,
                                    int64_t K) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (seq->finalized) return NVFP4_ERR_STATE;
    Job job;
    const int st = prepare_grouped(a_packed, a_scales, b_packed, b_scales, row_offsets, groups,
                                   alpha, out, M, N, K, NVFP4_PATH_AUTO, &job);
    return add_job(seq, st, job);
}

int nvfp4_sequence_add_quantize(nvfp4_sequence_t seq, const float* x, int64_t rows, int64_t K,
                                int64_t ld, void* packed_codes, void* packed_scales) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (seq->finalized) return NVFP4_ERR_STATE;
    Job job;
    const int st = prepare_quantize(x, false, rows, K, ld, packed_codes, packed_scales, &job);
    return add_job(seq, st, job);
}

int nvfp4_sequence_add_gemm_quantized(nvfp4_sequence_t seq, const void* x, int x_type,
                                      int64_t ldx, const void* b_packed, const void* b_scales,
                                      float alpha, void* out, int64_t M, int64_t N, int64_t K) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (seq->finalized) return NVFP4_ERR_STATE;
    Job job;
    const int st = prepare_gemm_quantized(x, x_type, ldx, b_packed, b_scales, alpha, out, M, N, K,
                                          &job);
    return add_job(seq, st, job);
}

int nvfp4_sequence_add_quantize_bf16(nvfp4_sequence_t seq, const void* x, int64_t rows, int64_t K,
                                     int64_t ld, void* packed_codes, void* packed_scales) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (seq->finalized) return NVFP4_ERR_STATE;
    Job job;
    const int st = prepare_quantize(x, true, rows, K, ld, packed_codes, packed_scales, &job);
    return add_job(seq, st, job);
}

int nvfp4_sequence_finalize(nvfp4_sequence_t seq) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (seq->finalized) return NVFP4_ERR_STATE;
    if (seq->jobs.empty()) return NVFP4_ERR_INVALID_VALUE;
    int device = 0;
    int st = current_device(&device);
    if (st != NVFP4_OK) return st;
    seq->device = device;
    // one workspace serves every call: they run one after another
    size_t floats = 0, flagged = 0, counters = 0;
    for (const Job& job : seq->jobs) {
        floats = job.floats > floats ? job.floats : floats;
        flagged = job.flagged > flagged ? job.flagged : flagged;
        counters = job.counters > counters ? job.counters : counters;
        // resolve every device query the launch makes before the capture
        if (job.kind == JOB_GEMM && job.plan.path == NVFP4_PATH_TILE &&
            resident_tiles(job.plan.cfg, device) <= 0)
            return NVFP4_ERR_HIP;
    }
    // zero-filled once, synchronously: counters and flagged words start clear
    auto alloc = [&](auto** p, size_t n) -> int {
        if (!n) return (int)NVFP4_OK;
        const size_t bytes = n * sizeof(**p);
        if (hipMalloc(p, bytes) != hipSuccess) return (int)NVFP4_ERR_ALLOC;
        return hipMemset(*p, 0, bytes) == hipSuccess ? (int)NVFP4_OK : (int)NVFP4_ERR_HIP;
    };
    st = alloc(&seq->ws.partials, floats);
    if (st == NVFP4_OK) st = alloc(&seq->ws.flagged, flagged);
    if (st == NVFP4_OK) st = alloc(&seq->ws.counters, counters);
    // the fills are complete before any launch of the sequence, on any stream
    if (st == NVFP4_OK && hipDeviceSynchronize() != hipSuccess) st = NVFP4_ERR_HIP;
    if (st != NVFP4_OK) {
        release(seq);
        return st;
    }
    st = capture(seq);
    if (st != NVFP4_OK) {
        release(seq);
        return st;
    }
    seq->finalized = true;
    return NVFP4_OK;
}

int nvfp4_sequence_launch(nvfp4_sequence_t seq, void* stream) {
    if (!seq) return NVFP4_ERR_INVALID_VALUE;
    if (!seq->finalized) return NVFP4_ERR_STATE;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return NVFP4_ERR_HIP;
    if (device != seq->device) return NVFP4_ERR_INVALID_VALUE;
    return hipGraphLaunch(seq->exec, static_cast<hipStream_t>(stream)) == hipSuccess
               ? NVFP4_OK
               : NVFP4_ERR_HIP;
}

int nvfp4_sequence_destroy(nvfp4_sequence_t seq) {
    if (!seq) return NVFP4_OK;
    release(seq);
    delete seq;
    return NVFP4_OK;
}

}  // extern "C"
