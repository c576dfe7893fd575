// nvfp4_api.cpp -- host side of the NVFP4 block-scaled GEMM library:
// argument validation, the canonical <-> packed layout transform, path and
// split-K planning, the per-(device, stream) split-K workspace, and launch.
//
// The operation and its argument rules are those of include/nvfp4.h: C =
// alpha * (A . B^T) on E2M1 codes with one E4M3 scale per 16 elements and a
// bfloat16 output ("Peeling the Kernel Onion", sections "The Benchmark
// Design" and "The Chain of Reasoning"); K must be a multiple of the block
// size, and mismatched operands are an error, not a silent result ("The
// SM120 FP4 Kernel Disaster", section "The Bash Command").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>

#include "nvfp4.h"
#include "nvfp4_internal.h"

using namespace nvfp4;

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every index in range of the kernels' int math

bool valid_rows_k(int64_t rows, int64_t K) {
    return rows >= 1 && rows <= kMaxDim && K >= 16 && K <= kMaxDim && (K % 16) == 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
    uint32_t* counters = nullptr;
    size_t counter_count = 0;
};

std::map<std::pair<int, void*>, Workspace> g_ws;

// Makes sure the workspace of (device, stream) can hold the request.  Growing
// it frees the old buffers (hipFree waits for work that may still use them)
// and zero-fills the new counters; this happens only when a larger shape is
// seen for the first time on that stream.
int get_workspace(int device, void* stream, size_t floats, size_t counters, Workspace** out) {
    std::lock_guard<std::mutex> lk(g_mu);
    Workspace& ws = g_ws[{device, stream}];
    if (floats > ws.partial_floats) {
        if (ws.partials) (void)hipFree(ws.partials);
        ws.partials = nullptr;
        ws.partial_floats = 0;
        if (hipMalloc(&ws.partials, floats * sizeof(float)) != hipSuccess) return NVFP4_ERR_ALLOC;
        ws.partial_floats = floats;
    }
    if (counters > ws.counter_count) {
        if (ws.counters) (void)hipFree(ws.counters);
        ws.counters = nullptr;
        ws.counter_count = 0;
        if (hipMalloc(&ws.counters, counters * sizeof(uint32_t)) != hipSuccess) return NVFP4_ERR_ALLOC;
        if (hipMemset(ws.counters, 0, counters * sizeof(uint32_t)) != hipSuccess) return NVFP4_ERR_HIP;
        ws.counter_count = counters;
    }
    *out = &ws;
    return NVFP4_OK;
}

// ---- planning ---------------------------------------------------------------

struct Plan {
    int path;
    int cfg;      // tile configuration (tile path)
    int split_k;
    int tiles_m, tiles_n;
};

constexpr int kCUs = 256;

Plan make_plan(int64_t M, int64_t N, int64_t K, int path, int split_req) {
    Plan p{};
    const int64_t P = num_panels(K);
    const int steps = (int)(P / 2);
    if (path == NVFP4_PATH_AUTO && M <= 4) path = NVFP4_PATH_GEMV;
    if (path == NVFP4_PATH_AUTO && M <= 16) path = NVFP4_PATH_SKINNY;
    p.path = path;
    if (path == NVFP4_PATH_GEMV) {
        p.split_k = 1;
        p.tiles_m = 1;
        p.tiles_n = (int)(round_up(N, kRowPad) / 4);
        return p;
    }
    if (path == NVFP4_PATH_SKINNY) {
        // One workgroup of kSkinnyWaves waves per 16 output columns covers the
        // whole K range: the split-K hand-off costs more than it saves once
        // there are 8 or more column groups (measured at 1x768x6144 and
        // 16x256x6144).  Fewer groups split K (each wave keeps at least one
        // 128-element work unit).
        const int64_t groups = round_up(N, kRowPad) / 16;
        int s = split_req;
        if (s <= 0) {
            s = (int)((8 + groups - 1) / groups);
            const int cap = steps / kSkinnyWaves;
            if (s > cap) s = cap;
        }
        if (s > steps) s = steps;
        p.split_k = s < 1 ? 1 : s;
        p.tiles_m = 1;
        p.tiles_n = (int)groups;
        return p;
    }
    if (path == NVFP4_PATH_AUTO) {
        // Large shapes whose 256 x 256 tiles nearly fill the machine use the
        // LDS-fed tile kernel; the rest use the kernel whose waves split K.
        const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
        path = t256 >= (3 * kCUs) / 4 ? NVFP4_PATH_TILE : NVFP4_PATH_WSPLIT;
        p.path = path;
    }
    if (path == NVFP4_PATH_WSPLIT) {
        const int cfg = WSPLIT_64x64;
        const TileShape s = wsplit_shape(cfg);
        p.cfg = cfg;
        p.tiles_m = (int)((M + s.bm - 1) / s.bm);
        p.tiles_n = (int)((N + s.bn - 1) / s.bn);
        const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
        int sk = split_req;
        if (sk <= 0) {
            // A workgroup (8 waves, ~236 VGPRs each) occupies a whole CU, so
            // split K across workgroups only while every workgroup still has
            // a CU of its own (a second round of workgroups costs more than
            // the split saves), keeping at least one panel per wave.
            sk = 1;
            while (tiles * (sk + 1) <= kCUs && (int64_t)(sk + 1) * 8 <= 2 * steps) ++sk;
        }
        if (sk > steps) sk = steps;
        p.split_k = sk < 1 ? 1 : sk;
        return p;
    }
    // Tile path: largest tile that still gives a reasonably full machine,
    // then split K until there are about two workgroups per CU.
    int cfg = TILE_256x256;
    for (int c : {TILE_256x256, TILE_128x128, TILE_64x64}) {
        const TileShape s = tile_shape(c);
        const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
        cfg = c;
        if (tiles >= kCUs) break;
    }
    const TileShape s = tile_shape(cfg);
    p.cfg = cfg;
    p.tiles_m = (int)((M + s.bm - 1) / s.bm);
    p.tiles_n = (int)((N + s.bn - 1) / s.bn);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    int sk = split_req;
    if (sk <= 0) {
        sk = 1;
        while (tiles * sk < kCUs && sk * 2 <= steps / 2) sk *= 2;
    }
    if (sk > steps) sk = steps;
    p.split_k = sk < 1 ? 1 : sk;
    return p;
}

int run_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
             const void* b_scales, float alpha, void* out, int64_t M, int64_t N, int64_t K,
             int path, int split_k, void* stream) {
    if (!a_packed || !a_scales || !b_packed || !b_scales || !out) return NVFP4_ERR_INVALID_VALUE;
    if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim) return NVFP4_ERR_INVALID_VALUE;
    if (!valid_rows_k(1, K)) return NVFP4_ERR_INVALID_VALUE;
    if (path < NVFP4_PATH_AUTO || path > NVFP4_PATH_GEMV || split_k < 0)
        return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(a_packed) || !aligned16(a_scales) || !aligned16(b_packed) ||
        !aligned16(b_scales) || !aligned16(out))
        return NVFP4_ERR_MISALIGNED;
    if (path == NVFP4_PATH_SKINNY && M > 16) return NVFP4_ERR_UNSUPPORTED;
    if (path == NVFP4_PATH_GEMV && M > 4) return NVFP4_ERR_UNSUPPORTED;

    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return NVFP4_ERR_HIP;
    const int dst = check_device(device);
    if (dst != NVFP4_OK) return dst;

    const Plan plan = make_plan(M, N, K, path, split_k);
    if (plan.path == NVFP4_PATH_TILE) {
        // the tile kernel addresses each packed operand with 32-bit offsets
        const int64_t P = num_panels(K);
        const int64_t limit = (int64_t)1 << 31;
        if (P * round_up(M, kRowPad) * kPanelCodeBytes >= limit ||
            P * round_up(N, kRowPad) * kPanelCodeBytes >= limit)
            return NVFP4_ERR_UNSUPPORTED;
    }
    GemmArgs a{};
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

    const size_t floats = plan.path == NVFP4_PATH_GEMV     ? 0
                          : plan.path == NVFP4_PATH_SKINNY ? skinny_partial_floats(a)
                          : plan.path == NVFP4_PATH_WSPLIT ? wsplit_partial_floats(plan.cfg, a)
                                                           : tile_partial_floats(plan.cfg, a);
    const size_t counters = plan.path == NVFP4_PATH_GEMV     ? 0
                            : plan.path == NVFP4_PATH_SKINNY ? skinny_counters(a)
                                                             : tile_counters(plan.cfg, a);
    if (floats || counters) {
        Workspace* ws = nullptr;
        const int wst = get_workspace(device, stream, floats, counters, &ws);
        if (wst != NVFP4_OK) return wst;
        a.partials = ws->partials;
        a.counters = ws->counters;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = plan.path == NVFP4_PATH_GEMV     ? launch_gemv(a, s)
                         : plan.path == NVFP4_PATH_SKINNY ? launch_skinny(a, s)
                         : plan.path == NVFP4_PATH_WSPLIT ? launch_wsplit(plan.cfg, a, s)
                                                          : launch_tile(plan.cfg, a, device, s);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace

extern "C" {

const char* nvfp4_status_string(int status) {
    switch (status) {
        case NVFP4_OK: return "success";
        case NVFP4_ERR_INVALID_VALUE: return "invalid value (sizes, K % 16, null pointer or option)";
        case NVFP4_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case NVFP4_ERR_UNSUPPORTED: return "unsupported device or path for this shape";
        case NVFP4_ERR_HIP: return "HIP runtime error";
        case NVFP4_ERR_ALLOC: return "workspace allocation failed";
        default: return "unknown status";
    }
}

int nvfp4_version(void) { return 100; }

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
    return check_device(device);
}

void nvfp4_shutdown(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    int current = 0;
    (void)hipGetDevice(&current);
    for (auto& kv : g_ws) {
        (void)hipSetDevice(kv.first.first);
        if (kv.second.partials) (void)hipFree(kv.second.partials);
        if (kv.second.counters) (void)hipFree(kv.second.counters);
    }
    (void)hipSetDevice(current);
    g_ws.clear();
}

int nvfp4_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
               const void* b_scales, float alpha, void* out, int64_t M, int64_t N, int64_t K,
               void* stream) {
    return run_gemm(a_packed, a_scales, b_packed, b_scales, alpha, out, M, N, K,
                    NVFP4_PATH_AUTO, 0, stream);
}

int nvfp4_gemm_with_path(const void* a_packed, const void* a_scales, const void* b_packed,
                         const void* b_scales, float alpha, void* out, int64_t M, int64_t N,
                         int64_t K, int path, int split_k, void* stream) {
    return run_gemm(a_packed, a_scales, b_packed, b_scales, alpha, out, M, N, K, path, split_k,
                    stream);
}

int nvfp4_quantize(const float* x, int64_t rows, int64_t K, int64_t ld, void* packed_codes,
                   void* packed_scales, void* stream) {
    if (!x || !packed_codes || !packed_scales || !valid_rows_k(rows, K) || ld < K || ld % 4 != 0)
        return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(x) || !aligned16(packed_codes) || !aligned16(packed_scales))
        return NVFP4_ERR_MISALIGNED;
    const int64_t Rp = round_up(rows, kRowPad);
    const int64_t P = num_panels(K);
    if (Rp * 16 > INT32_MAX || P > 65535) return NVFP4_ERR_INVALID_VALUE;  // grid size
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return NVFP4_ERR_HIP;
    const int dst = check_device(device);
    if (dst != NVFP4_OK) return dst;
    QuantArgs a{};
    a.x = x;
    a.codes = static_cast<uint8_t*>(packed_codes);
    a.scales = static_cast<uint8_t*>(packed_scales);
    a.ld = ld;
    a.rows = (int)rows;
    a.K = (int)K;
    a.Rp = (int)Rp;
    a.P = (int)P;
    const hipError_t e = launch_quantize(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_grouped_gemm(const void* a_packed, const void* a_scales, const void* b_packed,
                       const void* b_scales, const int32_t* row_offsets, int64_t groups,
                       float alpha, void* out, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!a_packed || !a_scales || !b_packed || !b_scales || !row_offsets || !out)
        return NVFP4_ERR_INVALID_VALUE;
    if (M < 0 || N < 1 || M > kMaxDim || N > kMaxDim || groups < 1 || !valid_rows_k(1, K))
        return NVFP4_ERR_INVALID_VALUE;
    const int64_t Np = round_up(N, kRowPad);
    if (groups * (Np / 16) > INT32_MAX) return NVFP4_ERR_INVALID_VALUE;
    if (!aligned16(a_packed) || !aligned16(a_scales) || !aligned16(b_packed) ||
        !aligned16(b_scales) || !aligned16(out) || (reinterpret_cast<uintptr_t>(row_offsets) & 3u))
        return NVFP4_ERR_MISALIGNED;
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return NVFP4_ERR_HIP;
    const int dst = check_device(device);
    if (dst != NVFP4_OK) return dst;
    if (M == 0) return NVFP4_OK;  // no rows: nothing to compute or write

    GroupedArgs a{};
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
    const hipError_t e = launch_grouped(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

int nvfp4_plan(int64_t M, int64_t N, int64_t K, int* path, int* split_k, int* tile_m,
               int* tile_n) {
    if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim || !valid_rows_k(1, K))
        return NVFP4_ERR_INVALID_VALUE;
    const Plan p = make_plan(M, N, K, NVFP4_PATH_AUTO, 0);
    if (path) *path = p.path;
    if (split_k) *split_k = p.split_k;
    const TileShape s = p.path == NVFP4_PATH_GEMV     ? TileShape{4, 1}
                        : p.path == NVFP4_PATH_SKINNY ? TileShape{16, 16}
                        : p.path == NVFP4_PATH_WSPLIT ? wsplit_shape(p.cfg)
                                                      : tile_shape(p.cfg);
    if (tile_m) *tile_m = s.bm;
    if (tile_n) *tile_n = s.bn;
    return NVFP4_OK;
}

}  // extern "C"
