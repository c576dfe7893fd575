// nvfp4_plan.cpp -- launch planning for the NVFP4 GEMM: which kernel path,
// which output tile and how many K slices a shape gets.
//
// Two sources, in this order (include/nvfp4.h, "Tuned plan table"):
//   1. a table of measured choices, loaded from a JSON file written by an
//      offline sweep (the pages' GEMM library autotunes tile configurations
//      per shape and lost or never saved the results: "The SM120 FP4 Kernel
//      Disaster", Finding 3; "The Multi-Pronged Investigation", Task 2);
//   2. the library's own rules, from the shape and the GPU's 256 CUs.
// Any plan computes the same GEMM; the choice changes only speed and the
// order of the FP32 additions.
#include "nvfp4_plan.h"

#include <cerrno>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "nvfp4.h"
#include "nvfp4_internal.h"

#ifndef NVFP4_BUILD_ID
#define NVFP4_BUILD_ID "unknown"
#endif

namespace nvfp4 {
namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;

// ---- tuned table --------------------------------------------------------------

struct Choice {
    int path, tile, split_k;
};

// (N, K) -> (M -> choice)
using Table = std::map<std::pair<int64_t, int64_t>, std::map<int64_t, Choice>>;

std::mutex g_table_mu;
std::shared_ptr<const Table> g_table;  // null: no table loaded

std::shared_ptr<const Table> current_table() {
    std::lock_guard<std::mutex> lk(g_table_mu);
    return g_table;
}

// The entry for (M, N, K): exact shape, else the same N and K with the
// smallest M' >= M, provided M' <= 2 M.
bool lookup(int64_t M, int64_t N, int64_t K, Choice* out) {
    const std::shared_ptr<const Table> t = current_table();
    if (!t) return false;
    const auto nk = t->find({N, K});
    if (nk == t->end()) return false;
    const auto it = nk->second.lower_bound(M);
    if (it == nk->second.end() || it->first > 2 * M) return false;
    *out = it->second;
    return true;
}

bool tile_allowed(int path, int tile) {
    switch (path) {
        case NVFP4_PATH_AUTO:
        case NVFP4_PATH_SKINNY:
        case NVFP4_PATH_GEMV: return tile == 0;
        case NVFP4_PATH_TILE: return tile == 0 || tile == 64 || tile == 128 || tile == 256;
        case NVFP4_PATH_WSPLIT: return tile == 0 || tile == 16 || tile == 32 || tile == 64 || tile == 128;
        default: return false;
    }
}

// ---- a small strict JSON reader (RFC 8259 values; no extensions) -------------

struct JValue {
    enum Kind { Null, Bool, Number, String, Array, Object } kind = Null;
    bool b = false;
    double num = 0.0;
    std::string str;
    std::vector<JValue> items;                            // Array
    std::vector<std::pair<std::string, JValue>> members;  // Object, in file order
    // Last member named `key` (a later duplicate wins), or null.
    const JValue* get(const char* key) const {
        const JValue* v = nullptr;
        for (const auto& m : members)
            if (m.first == key) v = &m.second;
        return v;
    }
};

class JReader {
  public:
    JReader(const char* p, const char* e) : p_(p), e_(e) {}
    bool parse(JValue& v) {
        if (!value(v, 0)) return false;
        ws();
        return p_ == e_;
    }

  private:
    const char* p_;
    const char* e_;
    static constexpr int kMaxDepth = 32;

    void ws() {
        while (p_ < e_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
    }
    bool peek(char c) const { return p_ < e_ && *p_ == c; }
    bool literal(const char* s) {
        const size_t n = std::strlen(s);
        if ((size_t)(e_ - p_) < n || std::memcmp(p_, s, n) != 0) return false;
        p_ += n;
        return true;
    }
    bool value(JValue& v, int depth) {
        if (depth > kMaxDepth) return false;
        ws();
        if (p_ >= e_) return false;
        switch (*p_) {
            case '{': return object(v, depth);
            case '[': return array(v, depth);
            case '"': v.kind = JValue::String; return string(v.str);
            case 't': v.kind = JValue::Bool; v.b = true; return literal("true");
            case 'f': v.kind = JValue::Bool; v.b = false; return literal("false");
            case 'n': v.kind = JValue::Null; return literal("null");
            default: v.kind = JValue::Number; return number(v.num);
        }
    }
    bool object(JValue& v, int depth) {
        v.kind = JValue::Object;
        ++p_;  // '{'
        ws();
        if (peek('}')) { ++p_; return true; }
        for (;;) {
            ws();
            std::string key;
            if (!peek('"') || !string(key)) return false;
            ws();
            if (!peek(':')) return false;
            ++p_;
            JValue m;
            if (!value(m, depth + 1)) return false;
            v.members.emplace_back(std::move(key), std::move(m));
            ws();
            if (peek(',')) { ++p_; continue; }
            if (peek('}')) { ++p_; return true; }
            return false;
        }
    }
    bool array(JValue& v, int depth) {
        v.kind = JValue::Array;
        ++p_;  // '['
        ws();
        if (peek(']')) { ++p_; return true; }
        for (;;) {
            JValue item;
            if (!value(item, depth + 1)) return false;
            v.items.push_back(std::move(item));
            ws();
            if (peek(',')) { ++p_; continue; }
            if (peek(']')) { ++p_; return true; }
            return false;
        }
    }
    static int hex(char c) {
        if (c >= '0' && c <= '9') return c - '0';
        if (c >= 'a' && c <= 'f') return c - 'a' + 10;
        if (c >= 'A' && c <= 'F') return c - 'A' + 10;
        return -1;
    }
    bool string(std::string& out) {
        ++p_;  // opening quote
        while (p_ < e_) {
            const char c = *p_++;
            if (c == '"') return true;
            if ((unsigned char)c < 0x20) return false;  // control characters must be escaped
            if (c != '\\') { out.push_back(c); continue; }
            if (p_ >= e_) return false;
            const char esc = *p_++;
            switch (esc) {
                case '"': case '\\': case '/': out.push_back(esc); break;
                case 'b': out.push_back('\b'); break;
                case 'f': out.push_back('\f'); break;
                case 'n': out.push_back('\n'); break;
                case 'r': out.push_back('\r'); break;
                case 't': out.push_back('\t'); break;
                case 'u': {
                    if (e_ - p_ < 4) return false;
                    unsigned cp = 0;
                    for (int i = 0; i < 4; ++i) {
                        const int h = hex(p_[i]);
                        if (h < 0) return false;
                        cp = cp * 16 + (unsigned)h;
                    }
                    p_ += 4;
                    // UTF-8 of the code unit (the table's keys and names are
                    // ASCII; other text only has to survive)
                    if (cp < 0x80) {
                        out.push_back((char)cp);
                    } else if (cp < 0x800) {
                        out.push_back((char)(0xC0 | (cp >> 6)));
                        out.push_back((char)(0x80 | (cp & 0x3F)));
                    } else {
                        out.push_back((char)(0xE0 | (cp >> 12)));
                        out.push_back((char)(0x80 | ((cp >> 6) & 0x3F)));
                        out.push_back((char)(0x80 | (cp & 0x3F)));
                    }
                    break;
                }
                default: return false;
            }
        }
        return false;  // unterminated
    }
    // -? (0 | [1-9][0-9]*) (. [0-9]+)? ([eE] [+-]? [0-9]+)?
    bool number(double& d) {
        const char* s = p_;
        const char* q = p_;
        auto digits = [&]() {
            const char* t = q;
            while (q < e_ && *q >= '0' && *q <= '9') ++q;
            return q > t;
        };
        if (q < e_ && *q == '-') ++q;
        if (q < e_ && *q == '0') {
            ++q;
        } else if (!digits()) {
            return false;
        }
        if (q < e_ && *q == '.') {
            ++q;
            if (!digits()) return false;
        }
        if (q < e_ && (*q == 'e' || *q == 'E')) {
            ++q;
            if (q < e_ && (*q == '+' || *q == '-')) ++q;
            if (!digits()) return false;
        }
        const std::string text(s, q);
        errno = 0;
        d = std::strtod(text.c_str(), nullptr);
        if (errno == ERANGE && std::isinf(d)) return false;
        p_ = q;
        return true;
    }
};

bool read_file(const char* path, std::string* out) {
    FILE* f = std::fopen(path, "rb");
    if (!f) return false;
    char buf[65536];
    size_t n;
    while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) {
        out->append(buf, n);
        if (out->size() > ((size_t)64 << 20)) {  // no plan table is this large
            std::fclose(f);
            return false;
        }
    }
    const bool ok = !std::ferror(f);
    std::fclose(f);
    return ok;
}

// Integer member `key` of `obj` in [lo, hi].
bool get_int(const JValue& obj, const char* key, int64_t lo, int64_t hi, int64_t* out) {
    const JValue* v = obj.get(key);
    if (!v || v->kind != JValue::Number || !std::isfinite(v->num)) return false;
    if (v->num != std::floor(v->num) || v->num < (double)lo || v->num > (double)hi) return false;
    *out = (int64_t)v->num;
    return true;
}

int path_of_name(const std::string& s) {
    if (s == "tile") return NVFP4_PATH_TILE;
    if (s == "skinny") return NVFP4_PATH_SKINNY;
    if (s == "wsplit") return NVFP4_PATH_WSPLIT;
    if (s == "gemv") return NVFP4_PATH_GEMV;
    return -1;
}

// One table entry, checked as nvfp4_gemm_with_plan would check it.
bool parse_entry(const JValue& e, int64_t* M, int64_t* N, int64_t* K, Choice* c) {
    if (e.kind != JValue::Object) return false;
    int64_t tile = 0, split = 0;
    if (!get_int(e, "M", 1, kMaxDim, M) || !get_int(e, "N", 1, kMaxDim, N) ||
        !get_int(e, "K", 16, kMaxDim, K) || (*K % 16) != 0)
        return false;
    const JValue* p = e.get("path");
    if (!p || p->kind != JValue::String) return false;
    c->path = path_of_name(p->str);
    if (c->path < 0) return false;
    if (e.get("tile") && !get_int(e, "tile", 0, 256, &tile)) return false;
    if (!get_int(e, "split_k", 1, 1 << 20, &split)) return false;
    if (!tile_allowed(c->path, (int)tile)) return false;
    if (c->path == NVFP4_PATH_SKINNY && *M > 64) return false;
    if (c->path == NVFP4_PATH_GEMV && *M > 4) return false;
    c->tile = (int)tile;
    c->split_k = (int)split;
    return true;
}

// ---- the library's rules ----------------------------------------------------

void plan_skinny(int64_t M, int64_t N, int steps, int split_req, Plan* p) {
    // One workgroup of kSkinnyWaves waves per 16 output columns covers the
    // whole K range when A has one block of 16 rows: the split-K hand-off
    // costs more than it saves once there are 8 or more column groups
    // (measured at 1x768x6144 and 16x256x6144); fewer groups split K (each
    // wave keeping at least one 128-element work unit).  With two to four
    // row blocks every workgroup decodes 2-4 fragments of A per unit, and
    // for up to 64 column groups K is split 3 ways (two blocks) or 4 ways
    // (three or four): 32 x 256..768 x 6144 6.3 -> 5.3-5.6 us, 64 x
    // 256..768 x 6144 7.6-7.8 -> 6.1-6.6 us; with more groups, two K slices
    // from three blocks on (64 x 2048 x 6144).
    const int64_t groups = round_up(N, kRowPad) / 16;
    int s = split_req;
    if (s <= 0) {
        if (M > 16 && groups <= 64) {
            s = M <= 32 ? 3 : 4;
            const int cap = steps / 4;  // at least four K steps per workgroup
            if (s > cap) s = cap;
        } else {
            s = (int)((8 + groups - 1) / groups);
            if (M > 32 && s < 2) s = 2;
            const int cap = steps / kSkinnyWaves;
            if (s > cap) s = cap;
        }
    }
    if (s > steps) s = steps;
    if (s > kSkinnyWaves) s = kSkinnyWaves;  // the last arrival fetches one split per wave
    p->split_k = s < 1 ? 1 : s;
    p->tiles_m = 1;
    p->tiles_n = (int)groups;
}

// Estimated device time (us, beyond the per-call floor) of the mid-size
// kernel with configuration `cfg` and `s` K slices.  Measured on an MI355X
// at M = 1..4096, N = 256..8192, K = 2048..16384 (graph replays): a tile
// costs about kWsplitPanelUs per 64-element K panel, the same for 1 to 256
// tiles; more tiles than CUs take further rounds; a split-K hand-off between
// workgroups (a ticket and the round trip of the partial tiles through
// memory) costs about 2 + s / 4 us.
constexpr double kWsplitPanelUs[4] = {0.115, 0.2, 0.071, 0.038};  // by WsplitConfig
double wsplit_estimate(int cfg, int64_t M, int64_t N, int steps, int s) {
    const TileShape t = wsplit_shape(cfg);
    const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const int64_t rounds = (tiles * s + kCUs - 1) / kCUs;
    return kWsplitPanelUs[cfg] * (2.0 * steps) * (double)rounds / s + (s > 1 ? 2.0 + 0.25 * s : 0.0);
}

// tile: 0 (choose), 16 (32 x 32), 32 (64 x 32), 64 (64 x 64) or 128 (128 x 64).
void plan_wsplit(int64_t M, int64_t N, int steps, int tile, int split_req, Plan* p) {
    int cfg = tile == 128 ? WSPLIT_128x64 : tile == 64 ? WSPLIT_64x64
            : tile == 32 ? WSPLIT_64x32 : WSPLIT_32x32;
    if (tile == 0) {
        // From the largest tile down, a smaller tile only where it is
        // estimated at least 10% faster without splitting K.
        double best = 0.0;
        bool first = true;
        for (int c : {WSPLIT_128x64, WSPLIT_64x64, WSPLIT_64x32, WSPLIT_32x32}) {
            const double e = wsplit_estimate(c, M, N, steps, 1);
            if (first || e < 0.9 * best) {
                cfg = c;
                best = e;
                first = false;
            }
        }
    }
    const TileShape s = wsplit_shape(cfg);
    p->cfg = cfg;
    p->tiles_m = (int)((M + s.bm - 1) / s.bm);
    p->tiles_n = (int)((N + s.bn - 1) / s.bn);
    const int64_t tiles = (int64_t)p->tiles_m * p->tiles_n;
    int sk = split_req;
    if (sk <= 0) {
        // Split K across workgroups only while every slice keeps a CU of its
        // own and at least one panel per wave, and only where that is
        // estimated at least 10% faster (long K on few tiles).
        sk = 1;
        double best = wsplit_estimate(cfg, M, N, steps, 1);
        for (int k = 2; k <= 8 && tiles * k <= kCUs && (int64_t)k * 8 <= 2 * steps; ++k) {
            const double e = wsplit_estimate(cfg, M, N, steps, k);
            if (e < 0.9 * best) {
                sk = k;
                best = e;
            }
        }
    }
    if (sk > steps) sk = steps;
    p->split_k = sk < 1 ? 1 : sk;
}

void plan_tile(int64_t M, int64_t N, int steps, int tile, int split_req, Plan* p) {
    int cfg = TILE_256x256;
    if (tile != 0) {
        cfg = tile == 256 ? TILE_256x256 : tile == 128 ? TILE_128x128 : TILE_64x64;
    } else {
        // largest tile that still gives a reasonably full machine
        for (int c : {TILE_256x256, TILE_128x128, TILE_64x64}) {
            const TileShape s = tile_shape(c);
            const int64_t tiles = ((M + s.bm - 1) / s.bm) * ((N + s.bn - 1) / s.bn);
            cfg = c;
            if (tiles >= kCUs) break;
        }
    }
    const TileShape s = tile_shape(cfg);
    p->cfg = cfg;
    p->tiles_m = (int)((M + s.bm - 1) / s.bm);
    p->tiles_n = (int)((N + s.bn - 1) / s.bn);
    const int64_t tiles = (int64_t)p->tiles_m * p->tiles_n;
    int sk = split_req;
    if (sk <= 0) {
        // split K until there are about as many workgroups as CUs
        sk = 1;
        while (tiles * sk < kCUs && sk * 2 <= steps / 2) sk *= 2;
    }
    if (sk > steps) sk = steps;
    p->split_k = sk < 1 ? 1 : sk;
    // 256 x 256 tiles run one workgroup per CU.  When the last round of a
    // persistent launch would be at most half full, its tiles go to a second
    // launch that splits their K range 2-4 ways (at least two K steps per
    // slice) over the CUs that round would leave idle: 384 tiles take about
    // 1.5 tile times instead of 2.
    if (p->split_k == 1 && cfg == TILE_256x256 && tiles > kCUs) {
        const int64_t rem = tiles % kCUs;
        int64_t s2 = rem > 0 ? kCUs / rem : 0;
        if (s2 > 4) s2 = 4;
        if (s2 > steps / 2) s2 = steps / 2;
        if (rem > 0 && rem <= kCUs / 2 && s2 >= 2) {
            p->tail_tiles = (int)rem;
            p->tail_split = (int)s2;
        }
    }
}

}  // namespace

int make_plan(int64_t M, int64_t N, int64_t K, int path, int tile, int split_req, Plan* p) {
    if (!tile_allowed(path, tile)) return NVFP4_ERR_INVALID_VALUE;
    *p = Plan{};
    p->source = NVFP4_PLAN_HEURISTIC;
    Choice c;
    if (path == NVFP4_PATH_AUTO && split_req == 0 && lookup(M, N, K, &c)) {
        path = c.path;
        tile = c.tile;
        split_req = c.split_k;
        p->source = NVFP4_PLAN_TABLE;
    }
    const int steps = (int)(num_panels(K) / 2);
    if (path == NVFP4_PATH_AUTO) {
        // Measured on an MI355X over M = 1..16384 for N x K = 256 .. 8192 x
        // 6144 .. 8192 (device time per call):
        //  * the dot-product kernel wins only while the whole output is at
        //    most 2048 elements of one or two rows; beyond that the skinny
        //    kernel's 16-row MFMA blocks are faster, up to 16 rows while
        //    N <= 4096 and 32 rows while N <= 1024 (16 x 2048 x 6144: 4.4 us
        //    against 5.8 us on 32 x 32 tiles of the mid-size kernel; 16 x
        //    6144 x 6144: 6.7 against 5.9 us; 64 x 768: 6.6 against 5.8 us);
        //  * the LDS-fed tile kernel wins once its 256 x 256 tiles give about
        //    3/4 of a workgroup per CU, and with two K slices from half a
        //    workgroup per CU (4096 x 2048 x 6144: 88 us against 95 us on
        //    128 x 128 tiles);
        //  * below that the kernel whose waves split K wins, with the tile
        //    and K split its cost estimate picks (plan_wsplit): 6-16% faster
        //    than 128 x 128 tiles of the tile kernel split two ways at 192-511
        //    such tiles (2048 x 2048 x 6144: 49 against 55 us).
        const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
        if (M <= 2 && M * N <= 2048) {
            path = NVFP4_PATH_GEMV;
        } else if ((M <= 16 && N <= 4096) || (M <= 32 && N <= 1024)) {
            path = NVFP4_PATH_SKINNY;
        } else if (t256 >= kCUs / 2) {
            path = NVFP4_PATH_TILE;
            tile = 256;
            split_req = split_req ? split_req : (t256 >= (3 * kCUs) / 4 ? 1 : 2);
        } else {
            path = NVFP4_PATH_WSPLIT;
            tile = 0;
        }
    }
    p->path = path;
    switch (path) {
        case NVFP4_PATH_GEMV:
            p->split_k = 1;
            p->tiles_m = 1;
            p->tiles_n = (int)(round_up(N, kRowPad) / 4);
            break;
        case NVFP4_PATH_SKINNY: plan_skinny(M, N, steps, split_req, p); break;
        case NVFP4_PATH_WSPLIT: plan_wsplit(M, N, steps, tile, split_req, p); break;
        default: plan_tile(M, N, steps, tile, split_req, p); break;
    }
    return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

int nvfp4_plan(int64_t M, int64_t N, int64_t K, nvfp4_plan_t* plan) {
    if (!plan || M < 1 || N < 1 || M > kMaxDim || N > kMaxDim || K < 16 || K > kMaxDim ||
        (K % 16) != 0)
        return NVFP4_ERR_INVALID_VALUE;
    Plan p;
    const int st = make_plan(M, N, K, NVFP4_PATH_AUTO, 0, 0, &p);
    if (st != NVFP4_OK) return st;
    const TileShape s = p.path == NVFP4_PATH_GEMV     ? TileShape{4, 1}
                        : p.path == NVFP4_PATH_SKINNY ? TileShape{16, 16}
                        : p.path == NVFP4_PATH_WSPLIT ? wsplit_shape(p.cfg)
                                                      : tile_shape(p.cfg);
    plan->path = p.path;
    plan->tile_m = s.bm;
    plan->tile_n = s.bn;
    plan->split_k = p.split_k;
    plan->tail_tiles = p.tail_tiles;
    plan->tail_split = p.tail_split;
    plan->source = p.source;
    return NVFP4_OK;
}

int nvfp4_plan_table_load(const char* json_path, int64_t* entries, int* same_build) {
    if (!json_path) return NVFP4_ERR_INVALID_VALUE;
    std::string text;
    if (!read_file(json_path, &text)) return NVFP4_ERR_INVALID_VALUE;
    JValue root;
    JReader reader(text.data(), text.data() + text.size());
    if (!reader.parse(root) || root.kind != JValue::Object) return NVFP4_ERR_INVALID_VALUE;
    const JValue* fmt = root.get("format");
    int64_t version = 0;
    if (!fmt || fmt->kind != JValue::String || fmt->str != "nvfp4-plan-table" ||
        !get_int(root, "version", 1, 1, &version))
        return NVFP4_ERR_INVALID_VALUE;
    const JValue* arch = root.get("arch");
    if (!arch || arch->kind != JValue::String) return NVFP4_ERR_INVALID_VALUE;
    if (arch->str != "gfx950") return NVFP4_ERR_UNSUPPORTED;
    const JValue* list = root.get("entries");
    if (!list || list->kind != JValue::Array) return NVFP4_ERR_INVALID_VALUE;
    auto table = std::make_shared<Table>();
    for (const JValue& e : list->items) {
        int64_t M, N, K;
        Choice c;
        if (!parse_entry(e, &M, &N, &K, &c)) return NVFP4_ERR_INVALID_VALUE;
        (*table)[{N, K}][M] = c;  // a later entry for the shape replaces an earlier one
    }
    const JValue* build = root.get("build");
    const bool same = build && build->kind == JValue::String && build->str == NVFP4_BUILD_ID;
    {
        std::lock_guard<std::mutex> lk(g_table_mu);
        g_table = std::move(table);
    }
    if (entries) *entries = (int64_t)list->items.size();
    if (same_build) *same_build = same ? 1 : 0;
    return NVFP4_OK;
}

void nvfp4_plan_table_clear(void) {
    std::lock_guard<std::mutex> lk(g_table_mu);
    g_table.reset();
}

const char* nvfp4_build_id(void) { return NVFP4_BUILD_ID; }

}  // extern "C"
