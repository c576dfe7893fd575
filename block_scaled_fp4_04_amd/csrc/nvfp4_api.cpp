// nvfp4_api.cpp -- host side of the NVFP4 block-scaled GEMM library:
// argument validation, the canonical <-> packed layout transform, the
// per-(device, stream) split-K workspace, and launch (planning is in
// nvfp4_plan.cpp).
//
// The operation and its argument rules are those of include/nvfp4.h: C =
// alpha * (A . B^T) on E2M1 codes with one E4M3 scale per 16 elements and a
// bfloat16 output ("Peeling the Kernel Onion", sections "The Benchmark
// Design" and "The Chain of Reasoning"); K must be a multiple of the block
// size, and mismatched operands are an error, not a silent result ("The
// SM120 FP4 Kernel Disaster", section "The Bash Command").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "nvfp4.h"
#include "nvfp4_host.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every index in range of the kernels' int math

bool valid_rows_k(int64_t rows, int64_t K) {
    return rows >= 1 && rows <= kMaxDim && K >= 16 && K <= kMaxDim && (K % 16) == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Poll budget of the two-way split-K hand-off given to the kernels
// (nvfp4_debug_set_handoff_polls changes it for tests).
std::atomic<uint32_t> g_handoff_polls{kHandoffPolls};

// ---- device checks -------------------------------------------------------

std::mutex g_mu;
std::map<int, int> g_device_ok;  // device -> status of the gfx950 check

int check_device(int device) {
    {
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_device_ok.find(device);
        if (it != g_device_ok.end()) return it->second;
    }
    hipDeviceProp_t prop;
    int st = NVFP4_OK;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) {
        st = NVFP4_ERR_HIP;
    } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        st = NVFP4_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    g_device_ok[device] = st;
    return st;
}

// ---- split-K workspace, one per (device, stream) ---------------------------

struct Workspace {
    float* partials = nullptr;
    size_t partial_floats = 0;
    uint64_t* flagged = nullptr;
    size_t flagged_words = 0;
    uint32_t* counters = nullptr;
    size_t counter_count = 0;
    // Buffers replaced by larger ones.  A graph captured on the stream may
    // still hold their addresses, so they stay allocated until
    // nvfp4_shutdown (freeing them would leave such a graph writing into
    // freed memory).
    std::vector<void*> retired;
};

std::map<std::pair<int, void*>, Workspace> g_ws;

bool capturing(void* stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) == hipSuccess &&
           cs != hipStreamCaptureStatusNone;
}

// Replaces *buf (holding *have elements) by an allocation of `need`
// elements if it is smaller, zero-filled on `stream` (so the fill is ordered
// before the kernels the caller enqueues next on that stream); the old
// buffer is retired.
template <typename T>
int grow(T** buf, size_t* have, size_t need, std::vector<void*>& retired, void* stream) {
    if (need <= *have) return NVFP4_OK;
    T* p = nullptr;
    if (hipMalloc(&p, need * sizeof(T)) != hipSuccess) return NVFP4_ERR_ALLOC;
    if (hipMemsetAsync(p, 0, need * sizeof(T), static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipFree(p);
        return NVFP4_ERR_HIP;
    }
    if (*buf) retired.push_back(*buf);
    *buf = p;
    *have = need;
    return NVFP4_OK;
}

// Makes sure the workspace of (device, stream) can hold the job's needs.
// Growing it allocates larger buffers and zero-fills them on the stream
// itself, ahead of the job's kernels (counters and flagged words must be
// clear before any kernel uses them; a fill on another stream could land
// after a kernel had published a word); the old buffers are retired, not
// freed (see Workspace::retired).  This happens only when a larger shape is
// seen for the first time on that stream, and never while the stream is
// being captured into a graph (NVFP4_ERR_CAPTURE: allocation and fills are
// not allowed there).
int get_workspace(int device, void* stream, const Job& job, WorkspacePtrs* out) {
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace& ws = g_ws[{device, stream}];
    if ((job.floats > ws.partial_floats || job.flagged > ws.flagged_words ||
         job.counters > ws.counter_count) &&
        capturing(stream))
        return NVFP4_ERR_CAPTURE;
    int st = grow(&ws.partials, &ws.partial_floats, job.floats, ws.retired, stream);
    if (st == NVFP4_OK) st = grow(&ws.flagged, &ws.flagged_words, job.flagged, ws.retired, stream);
    if (st == NVFP4_OK) st = grow(&ws.counters, &ws.counter_count, job.counters, ws.retired, stream);
    if (st != NVFP4_OK) return st;
    out->partials = ws.partials;
    out->flagged = ws.flagged;
    out->counters = ws.counters;
    return NVFP4_OK;
}

// Runs a prepared job eagerly on `stream` with that stream's workspace.
int run_job(const Job& job, void* stream) {
    int device = 0;
    const int dst = current_device(&device);
    if (dst != NVFP4_OK || job.empty) return dst;
    WorkspacePtrs ws;
    if (job.floats || job.flagged || job.counters) {
        const int wst = get_workspace(device, stream, job, &ws);
        if (wst != NVFP4_OK) return wst;
    }
    const hipError_t e = launch_job(job, device, ws, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace

// ---- jobs ---------------------------------------------------------------------

namespace nvfp4 {

int current_device(int* device) {
    if (hipGetDevice(device) != hipSuccess) return NVFP4_ERR_HIP;
    return check_device(*device);
}

int prepare_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
                 const void* b_scales, float alpha, void* out, int64_t M, int64_t N, int64_t K,
                 int path, int tile, int split_k, Job* job) {
    if (!a_packed || !a_scales || !b_packed || !b_scales || !out) return NVFP4_ERR_INVALID_VALUE;
    if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim) return NVFP4_ERR_INVALID_VALUE;
    if (!valid_rows_k(1, K)) return NVFP4_ERR_INVALID_VALUE;
    if (path < NVFP4_PATH_AUTO || path > NVFP4_PATH_GEMV || split_k < 0)
        return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(a_packed) || !aligned16(a_scales) || !aligned16(b_packed) ||
        !aligned16(b_scales) || !aligned16(out))
        return NVFP4_ERR_MISALIGNED;
    if (path == NVFP4_PATH_SKINNY && M > 64) return NVFP4_ERR_UNSUPPORTED;
    if (path == NVFP4_PATH_GEMV && M > 4) return NVFP4_ERR_UNSUPPORTED;

    *job = Job{};
    job->kind = JOB_GEMM;
    Plan& plan = job->plan;
    const int pst = make_plan(M, N, K, path, tile, split_k, &plan);
    if (pst != NVFP4_OK) return pst;
    if (plan.path == NVFP4_PATH_TILE || plan.path == NVFP4_PATH_WSPLIT) {
        // the tile and wsplit kernels address each packed operand with 32-bit offsets
        const int64_t P = num_panels(K);
        const int64_t limit = (int64_t)1 << 31;
        if (P * round_up(M, kRowPad) * kPanelCodeBytes >= limit ||
            P * round_up(N, kRowPad) * kPanelCodeBytes >= limit)
            return NVFP4_ERR_UNSUPPORTED;
    }
    GemmArgs& a = job->gemm;
    a.a_codes = static_cast<const uint8_t*>(a_packed);
    a.a_scales = static_cast<const uint8_t*>(a_scales);
    a.b_codes = static_cast<const uint8_t*>(b_packed);
    a.b_scales = static_cast<const uint8_t*>(b_scales);
    a.out = static_cast<uint16_t*>(out);
    a.alpha = alpha;
    a.M = (int)M;
    a.N = (int)N;
    a.Mp = (int)round_up(M, kRowPad);
    a.Np = (int)round_up(N, kRowPad);
    a.P = (int)(num_panels(K));
    a.split_k = plan.split_k;
    a.tiles_m = plan.tiles_m;
    a.tiles_n = plan.tiles_n;
    a.tile_begin = 0;
    a.tile_count = plan.tiles_m * plan.tiles_n;
    a.tail_tiles = plan.tail_tiles;
    a.tail_split = plan.tail_split;
    a.handoff_polls = g_handoff_polls.load(std::memory_order_relaxed);
    job->floats = plan.path == NVFP4_PATH_TILE     ? tile_partial_floats(plan.cfg, a)
                  : plan.path == NVFP4_PATH_WSPLIT ? wsplit_partial_floats(plan.cfg, a)
                                                   : 0;
    job->flagged = plan.path == NVFP4_PATH_SKINNY ? skinny_flagged_words(a) : 0;
    job->counters = plan.path == NVFP4_PATH_GEMV     ? 0
                    : plan.path == NVFP4_PATH_SKINNY ? skinny_counters(a)
                                                     : tile_counters(plan.cfg, a);
    return NVFP4_OK;
}

int prepare_grouped(const void* a_packed, const void* a_scales, const void* b_packed,
                    const void* b_scales, const int32_t* row_offsets, int64_t groups, float alpha,
                    void* out, int64_t M, int64_t N, int64_t K, int path, Job* job) {
    if (!a_packed || !a_scales || !b_packed || !b_scales || !row_offsets || !out)
        return NVFP4_ERR_INVALID_VALUE;
    if (path != NVFP4_PATH_AUTO && path != NVFP4_PATH_SKINNY && path != NVFP4_PATH_WSPLIT &&
        path != NVFP4_PATH_TILE)
        return NVFP4_ERR_INVALID_VALUE;
    if (M < 0 || N < 1 || M > kMaxDim || N > kMaxDim || groups < 1 || !valid_rows_k(1, K))
        return NVFP4_ERR_INVALID_VALUE;
    const int64_t Np = round_up(N, kRowPad);
    if (groups * (Np / 16) > INT32_MAX) return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(a_packed) || !aligned16(a_scales) || !aligned16(b_packed) ||
        !aligned16(b_scales) || !aligned16(out) || (reinterpret_cast<uintptr_t>(row_offsets) & 3u))
        return NVFP4_ERR_MISALIGNED;
    *job = Job{};
    job->empty = M == 0;  // no rows: nothing to compute or write
    const int64_t P = num_panels(K);
    const int64_t Mp = round_up(M, kRowPad);
    // Three kernels, by the average rows per group (measured with 32-256
    // experts of equal size, K = 6144): the grouped skinny kernel up to 32
    // rows, which it covers in one pass over B (256 experts, N = 256: 49
    // against 59 us for the mid-size kernel at 32 rows, 88 against 63 at
    // 40); the grouped mid-size kernel from kGroupedWsplitRows (at 128 rows
    // 121 against 190 us for the skinny and 246 for the tile kernel, N =
    // 256); the tile kernel with 256 x 256 tiles from kGroupedTileRows (at
    // 448 rows the mid-size kernel is still 6-7% faster at N = 256, 2048
    // and 6144, at 480-512 the tile kernel 0-4%).
    // The tile and mid-size kernels address A and each group's B with 32-bit
    // offsets; the mid-size kernel keeps a table of the groups in LDS.
    const bool offsets32 = P * Mp * kPanelCodeBytes < ((int64_t)1 << 31) &&
                           P * Np * kPanelCodeBytes < ((int64_t)1 << 31);
    const int64_t avg = M / groups;
    const int64_t tiles_n64 = (N + 63) / 64;
    const bool wsplit_ok = offsets32 && groups <= kGroupedWsplitMaxGroups &&
                           ((M + 63) / 64 + groups) * tiles_n64 <= INT32_MAX;
    int use = path;
    if (use == NVFP4_PATH_AUTO)
        use = (M > 0 && avg >= kGroupedTileRows && offsets32) ? NVFP4_PATH_TILE
              : (M > 0 && avg >= kGroupedWsplitRows && wsplit_ok) ? NVFP4_PATH_WSPLIT
                                                                  : NVFP4_PATH_SKINNY;
    if (use == NVFP4_PATH_WSPLIT) {
        if (!wsplit_ok) return NVFP4_ERR_UNSUPPORTED;
        job->kind = JOB_GROUPED_WSPLIT;
    }
    if (use == NVFP4_PATH_TILE) {
        if (!offsets32) return NVFP4_ERR_UNSUPPORTED;
        const int cfg = TILE_256x256;
        const TileShape ts = tile_shape(cfg);
        const int64_t tiles_m = (M + ts.bm - 1) / ts.bm + groups;  // bound: each group adds at most one partial block
        const int64_t tiles_n = (N + ts.bn - 1) / ts.bn;
        if (tiles_m * tiles_n > INT32_MAX) {
            if (path == NVFP4_PATH_TILE) return NVFP4_ERR_UNSUPPORTED;
        } else {
            job->kind = JOB_GROUPED_TILE;
            job->plan.path = NVFP4_PATH_TILE;
            job->plan.cfg = cfg;
            GemmArgs& g = job->gemm;
            g.a_codes = static_cast<const uint8_t*>(a_packed);
            g.a_scales = static_cast<const uint8_t*>(a_scales);
            g.b_codes = static_cast<const uint8_t*>(b_packed);
            g.b_scales = static_cast<const uint8_t*>(b_scales);
            g.out = static_cast<uint16_t*>(out);
            g.alpha = alpha;
            g.M = (int)M;
            g.N = (int)N;
            g.Mp = (int)Mp;
            g.Np = (int)Np;
            g.P = (int)P;
            g.split_k = 1;
            g.tiles_m = (int)tiles_m;
            g.tiles_n = (int)tiles_n;
            g.tile_begin = 0;
            g.tile_count = (int)(tiles_m * tiles_n);
            g.offsets = row_offsets;
            g.groups = (int)groups;
            g.handoff_polls = g_handoff_polls.load(std::memory_order_relaxed);
            return NVFP4_OK;
        }
    }
    if (job->kind != JOB_GROUPED_WSPLIT) job->kind = JOB_GROUPED;
    GroupedArgs& a = job->grouped;
    a.a_codes = static_cast<const uint8_t*>(a_packed);
    a.a_scales = static_cast<const uint8_t*>(a_scales);
    a.b_codes = static_cast<const uint8_t*>(b_packed);
    a.b_scales = static_cast<const uint8_t*>(b_scales);
    a.offsets = row_offsets;
    a.out = static_cast<uint16_t*>(out);
    a.alpha = alpha;
    a.M = (int)M;
    a.N = (int)N;
    a.Mp = (int)round_up(M, kRowPad);
    a.Np = (int)Np;
    a.P = (int)num_panels(K);
    a.G = (int)groups;
    return NVFP4_OK;
}

int prepare_quantize(const void* x, bool bf16, int64_t rows, int64_t K, int64_t ld,
                     void* packed_codes, void* packed_scales, Job* job) {
    // rows start on 16-byte boundaries: 4 fp32 or 8 bfloat16 values
    if (!x || !packed_codes || !packed_scales || !valid_rows_k(rows, K) || ld < K ||
        ld % (bf16 ? 8 : 4) != 0)
        return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(x) || !aligned16(packed_codes) || !aligned16(packed_scales))
        return NVFP4_ERR_MISALIGNED;
    const int64_t Rp = round_up(rows, kRowPad);
    const int64_t P = num_panels(K);
    if (Rp * 16 > INT32_MAX || P > 65535) return NVFP4_ERR_INVALID_VALUE;  // grid size
    *job = Job{};
    job->kind = JOB_QUANTIZE;
    QuantArgs& a = job->quant;
    a.x = x;
    a.bf16 = bf16;
    a.codes = static_cast<uint8_t*>(packed_codes);
    a.scales = static_cast<uint8_t*>(packed_scales);
    a.ld = ld;
    a.rows = (int)rows;
    a.K = (int)K;
    a.Rp = (int)Rp;
    a.P = (int)P;
    return NVFP4_OK;
}

int prepare_gemm_quantized(const void* x, int x_type, int64_t ldx, const void* b_packed,
                           const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                           int64_t K, Job* job) {
    if (!x || !b_packed || !b_scales || !out) return NVFP4_ERR_INVALID_VALUE;
    if (x_type != NVFP4_INPUT_F32 && x_type != NVFP4_INPUT_BF16) return NVFP4_ERR_INVALID_VALUE;
    const bool bf16 = x_type == NVFP4_INPUT_BF16;
    if (M < 1 || N < 1 || N > kMaxDim || !valid_rows_k(1, K) || ldx < K || ldx % (bf16 ? 8 : 4) != 0)
        return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(x) || !aligned16(b_packed) || !aligned16(b_scales) || !aligned16(out))
        return NVFP4_ERR_MISALIGNED;
    const int64_t P = num_panels(K);
    if (M > 4 || gemv_rows((int)M) * P * 64 > kGemvQuantElems) return NVFP4_ERR_UNSUPPORTED;
    *job = Job{};
    job->kind = JOB_GEMV_QUANT;
    GemvQuantArgs& g = job->gemvq;
    g.x = x;
    g.bf16 = bf16;
    g.ldx = ldx;
    g.b_codes = static_cast<const uint8_t*>(b_packed);
    g.b_scales = static_cast<const uint8_t*>(b_scales);
    g.out = static_cast<uint16_t*>(out);
    g.alpha = alpha;
    g.M = (int)M;
    g.N = (int)N;
    g.K = (int)K;
    g.Np = (int)round_up(N, kRowPad);
    g.P = (int)P;
    return NVFP4_OK;
}

hipError_t launch_job(const Job& job, int device, const WorkspacePtrs& ws, hipStream_t s) {
    if (job.empty) return hipSuccess;
    if (job.kind == JOB_GEMV_QUANT) return launch_gemv_quant(job.gemvq, s);
    if (job.kind == JOB_GROUPED) return launch_grouped(job.grouped, s);
    if (job.kind == JOB_GROUPED_TILE) return launch_grouped_tile(job.gemm, s);
    if (job.kind == JOB_GROUPED_WSPLIT) return launch_grouped_wsplit(job.grouped, s);
    if (job.kind == JOB_QUANTIZE) return launch_quantize(job.quant, s);
    GemmArgs a = job.gemm;
    a.partials = ws.partials;
    a.flagged = ws.flagged;
    a.counters = ws.counters;
    const Plan& plan = job.plan;
    return plan.path == NVFP4_PATH_GEMV     ? launch_gemv(a, s)
           : plan.path == NVFP4_PATH_SKINNY ? launch_skinny(a, s)
           : plan.path == NVFP4_PATH_WSPLIT ? launch_wsplit(plan.cfg, a, s)
                                            : launch_tile(plan.cfg, a, device, s);
}

}  // namespace nvfp4

extern "C" {

const char* nvfp4_status_string(int status) {
    switch (status) {
        case NVFP4_OK: return "success";
        case NVFP4_ERR_INVALID_VALUE: return "invalid value (sizes, K % 16, null pointer or option)";
        case NVFP4_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case NVFP4_ERR_UNSUPPORTED: return "unsupported device or path for this shape";
        case NVFP4_ERR_HIP: return "HIP runtime error";
        case NVFP4_ERR_ALLOC: return "workspace allocation failed";
        case NVFP4_ERR_CAPTURE: return "workspace needed while the stream is being captured";
        case NVFP4_ERR_STATE: return "call not allowed in the object's current state";
        case NVFP4_ERR_SCRATCH: return "the plan needs more split-K scratch than the static maximum";
        case NVFP4_ERR_DEVICE_FLAGS: return "a kernel raised a device error flag (see nvfp4_device_flags)";
        default: return "unknown status";
    }
}

int nvfp4_version(void) { return 10500; }

int nvfp4_packed_size(int64_t rows, int64_t K, size_t* code_bytes, size_t* scale_bytes) {
    if (!code_bytes || !scale_bytes || !valid_rows_k(rows, K)) return NVFP4_ERR_INVALID_VALUE;
    const int64_t Rp = round_up(rows, kRowPad);
    const int64_t P = num_panels(K);
    *code_bytes = (size_t)(P * Rp * kPanelCodeBytes);
    *scale_bytes = (size_t)(P * Rp * kPanelScaleBytes);
    return NVFP4_OK;
}

int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
               uint8_t* packed_codes, uint8_t* packed_scales) {
    if (!codes || !scales || !packed_codes || !packed_scales || !valid_rows_k(rows, K))
        return NVFP4_ERR_INVALID_VALUE;
    const int64_t Rp = round_up(rows, kRowPad);
    const int64_t P = num_panels(K);
    const int64_t rb = K / 2, rs = K / 16;  // canonical row strides
    for (int64_t p = 0; p < P; ++p) {
        for (int64_t r = 0; r < Rp; ++r) {
            uint8_t* dc = packed_codes + (p * Rp + r) * kPanelCodeBytes;
            uint8_t* ds = packed_scales + (p * Rp + r) * kPanelScaleBytes;
            const int64_t j0 = p * kPanelCodeBytes, b0 = p * kPanelScaleBytes;
            if (r >= rows) {
                std::memset(dc, 0, kPanelCodeBytes);
                std::memset(ds, 0, kPanelScaleBytes);
                continue;
            }
            // bytes of this panel that exist in the canonical row (0 in the
            // zero panels that round K up to whole steps)
            const int64_t nc = std::max<int64_t>(0, std::min<int64_t>(kPanelCodeBytes, rb - j0));
            const int64_t ns = std::max<int64_t>(0, std::min<int64_t>(kPanelScaleBytes, rs - b0));
            if (nc > 0) std::memcpy(dc, codes + r * rb + j0, (size_t)nc);
            if (nc < kPanelCodeBytes) std::memset(dc + nc, 0, (size_t)(kPanelCodeBytes - nc));
            if (ns > 0) std::memcpy(ds, scales + r * rs + b0, (size_t)ns);
            if (ns < kPanelScaleBytes) std::memset(ds + ns, 0, (size_t)(kPanelScaleBytes - ns));
        }
    }
    return NVFP4_OK;
}

int nvfp4_unpack(const uint8_t* packed_codes, const uint8_t* packed_scales, int64_t rows,
                 int64_t K, uint8_t* codes, uint8_t* scales) {
    if (!codes || !scales || !packed_codes || !packed_scales || !valid_rows_k(rows, K))
        return NVFP4_ERR_INVALID_VALUE;
    const int64_t Rp = round_up(rows, kRowPad);
    const int64_t P = num_panels(K);
    const int64_t rb = K / 2, rs = K / 16;
    for (int64_t p = 0; p < P; ++p) {
        for (int64_t r = 0; r < rows; ++r) {
            const uint8_t* sc = packed_codes + (p * Rp + r) * kPanelCodeBytes;
            const uint8_t* ss = packed_scales + (p * Rp + r) * kPanelScaleBytes;
            const int64_t j0 = p * kPanelCodeBytes, b0 = p * kPanelScaleBytes;
            const int64_t nc = std::max<int64_t>(0, std::min<int64_t>(kPanelCodeBytes, rb - j0));
            const int64_t ns = std::max<int64_t>(0, std::min<int64_t>(kPanelScaleBytes, rs - b0));
            if (nc > 0) std::memcpy(codes + r * rb + j0, sc, (size_t)nc);
            if (ns > 0) std::memcpy(scales + r * rs + b0, ss, (size_t)ns);
        }
    }
    return NVFP4_OK;
}

int nvfp4_init(int device) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess) return NVFP4_ERR_HIP;
    if (device < 0 || device >= count) return NVFP4_ERR_INVALID_VALUE;
    const int st = check_device(device);
    return st != NVFP4_OK ? st : noalloc_setup(device);
}

void nvfp4_shutdown(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int current = 0;
    (void)hipGetDevice(&current);
    for (auto& kv : g_ws) {
        (void)hipSetDevice(kv.first.first);
        if (kv.second.partials) (void)hipFree(kv.second.partials);
        if (kv.second.flagged) (void)hipFree(kv.second.flagged);
        if (kv.second.counters) (void)hipFree(kv.second.counters);
        for (void* p : kv.second.retired) (void)hipFree(p);
    }
    (void)hipSetDevice(current);
    g_ws.clear();
}

int nvfp4_device_flags(uint32_t* flags) {
    if (!flags) return NVFP4_ERR_INVALID_VALUE;
    int device = 0;
    const int st = current_device(&device);
    if (st != NVFP4_OK) return st;
    if (take_device_flags(flags) != hipSuccess) return NVFP4_ERR_HIP;
    return *flags ? NVFP4_ERR_DEVICE_FLAGS : NVFP4_OK;
}

int nvfp4_debug_set_handoff_polls(uint32_t polls) {
    g_handoff_polls.store(polls == 0xFFFFFFFFu ? kHandoffPolls : polls, std::memory_order_relaxed);
    return NVFP4_OK;
}

int nvfp4_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
               const void* b_scales, float alpha, void* out, int64_t M, int64_t N, int64_t K,
               void* stream) {
    return nvfp4_gemm_with_plan(a_packed, a_scales, b_packed, b_scales, alpha, out, M, N, K,
                                NVFP4_PATH_AUTO, 0, 0, stream);
}

int nvfp4_gemm_with_plan(const void* a_packed, const void* a_scales, const void* b_packed,
                         const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                         int64_t K, int path, int tile, int split_k, void* stream) {
    Job job;
    const int st = prepare_gemm(a_packed, a_scales, b_packed, b_scales, alpha, out, M, N, K, path,
                                tile, split_k, &job);
    return st != NVFP4_OK ? st : run_job(job, stream);
}

int nvfp4_quantize(const float* x, int64_t rows, int64_t K, int64_t ld, void* packed_codes,
                   void* packed_scales, void* stream) {
    Job job;
    const int st = prepare_quantize(x, false, rows, K, ld, packed_codes, packed_scales, &job);
    return st != NVFP4_OK ? st : run_job(job, stream);
}

int nvfp4_quantize_bf16(const void* x, int64_t rows, int64_t K, int64_t ld, void* packed_codes,
                        void* packed_scales, void* stream) {
    Job job;
    const int st = prepare_quantize(x, true, rows, K, ld, packed_codes, packed_scales, &job);
    return st != NVFP4_OK ? st : run_job(job, stream);
}

int nvfp4_gemm_quantized(const void* x, int x_type, int64_t ldx, const void* b_packed,
                         const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                         int64_t K, void* stream) {
    Job job;
    const int st = prepare_gemm_quantized(x, x_type, ldx, b_packed, b_scales, alpha, out, M, N, K,
                                          &job);
    return st != NVFP4_OK ? st : run_job(job, stream);
}

int nvfp4_grouped_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
                       const void* b_scales, const int32_t* row_offsets, int64_t groups,
                       float alpha, void* out, int64_t M, int64_t N, int64_t K, void* stream) {
    return nvfp4_grouped_gemm_with_plan(a_packed, a_scales, b_packed, b_scales, row_offsets,
                                        groups, alpha, out, M, N, K, NVFP4_PATH_AUTO, stream);
}

int nvfp4_grouped_gemm_with_plan(const void* a_packed, const void* a_scales,
                                 const void* b_packed, const void* b_scales,
                                 const int32_t* row_offsets, int64_t groups, float alpha,
                                 void* out, int64_t M, int64_t N, int64_t K, int path,
                                 void* stream) {
    Job job;
    const int st = prepare_grouped(a_packed, a_scales, b_packed, b_scales, row_offsets, groups,
                                   alpha, out, M, N, K, path, &job);
    return st != NVFP4_OK ? st : run_job(job, stream);
}

}  // extern "C"
