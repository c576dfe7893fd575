// nvfp4_internal.h -- launch arguments shared by the host library and the
// gfx950 kernels of the NVFP4 block-scaled GEMM (not part of the public ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// Packed operand geometry (see include/nvfp4.h, "Packed layout").
constexpr int kPanelK = 64;        // elements per panel
constexpr int kStepK = 128;        // K is padded to whole steps of two panels
constexpr int kPanelCodeBytes = 32;  // bytes of codes per row per panel
constexpr int kPanelScaleBytes = 4;  // scale bytes per row per panel
constexpr int kRowPad = 16;
constexpr int kSkinnyWaves = 16;    // waves per workgroup of the skinny kernel
constexpr int kCUs = 256;           // compute units of an MI355X (plans and grid sizes)

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
// Number of 64-element panels of a packed operand (always even).
inline int64_t num_panels(int64_t K) { return round_up(K, kStepK) / kPanelK; }

struct GemmArgs {
    const uint8_t* a_codes;   // [P][Mp][32]
    const uint8_t* a_scales;  // [P][Mp][4]
    const uint8_t* b_codes;   // [P][Np][32]
    const uint8_t* b_scales;  // [P][Np][4]
    uint16_t* out;            // [M][N] bfloat16 bits
    float* partials;          // split-K partial sums (tile, wsplit kernels; workspace), or null
    uint64_t* flagged;        // split-K partial sums with ready flags (skinny kernel), or null
    uint32_t* counters;       // split-K arrival counters (workspace), or null
    float alpha;
    int M, N;                 // logical output size
    int Mp, Np;               // padded row counts of the packed operands
    int P;                    // number of 64-element K panels (even)
    int split_k;              // number of K slices (>= 1)
    int tiles_m, tiles_n;     // output tiles along M and N (tile kernel)
    int tile_begin, tile_count;  // tiles [tile_begin, tile_begin + tile_count) of the
                                 // tiles_m x tiles_n grid this launch computes (tile kernel)
    int tail_tiles, tail_split;  // tile kernel without split-K: the last tail_tiles tiles
                                 // run in a second launch split tail_split ways along K
    const int32_t* offsets;   // grouped tile launch: [groups + 1] row offsets (device), else null
    int groups;               // grouped tile launch: number of groups (B holds one N x K operand each)
    uint32_t handoff_polls;   // tile kernel, two K slices: polls before the second workgroup
                              // gives up waiting for the first one's partial tile
};

// Polls of a two-way split-K hand-off before it gives up (each poll sleeps
// about 128 cycles, so the default is a fraction of a second; the partner
// workgroup is already running when the wait starts, so it never runs out in
// practice).
constexpr uint32_t kHandoffPolls = 1u << 22;

// Sticky error flags the kernels raise on the device (include/nvfp4.h,
// nvfp4_device_flags); bit values match NVFP4_FLAG_*.
constexpr uint32_t kFlagHandoff = 1u;

// Reads the flags of the current device (after synchronising it) and clears them.
hipError_t take_device_flags(uint32_t* flags);

// Tile configurations of the large-M kernel.
enum TileConfig { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x64 = 2 };

struct TileShape { int bm, bn; };
inline TileShape tile_shape(int cfg) {
    switch (cfg) {
        case TILE_256x256: return {256, 256};
        case TILE_128x128: return {128, 128};
        default: return {64, 64};
    }
}


// Workspace needs of a launch: FP32 partials, flagged 64-bit partial words,
// arrival counters.
size_t tile_partial_floats(int cfg, const GemmArgs& a);
size_t tile_counters(int cfg, const GemmArgs& a);
size_t skinny_flagged_words(const GemmArgs& a);
size_t skinny_counters(const GemmArgs& a);

// Mid-size kernel configurations (waves split K inside a workgroup), by
// output tile: rows of A x rows of B.
enum WsplitConfig { WSPLIT_64x64 = 0, WSPLIT_128x64 = 1, WSPLIT_64x32 = 2, WSPLIT_32x32 = 3 };
inline TileShape wsplit_shape(int cfg) {
    switch (cfg) {
        case WSPLIT_64x64: return TileShape{64, 64};
        case WSPLIT_64x32: return TileShape{64, 32};
        case WSPLIT_32x32: return TileShape{32, 32};
        default: return TileShape{128, 64};
    }
}
size_t wsplit_partial_floats(int cfg, const GemmArgs& a);

// Workgroups of a tile configuration resident on `device` at once (queried
// once per device and configuration; 0 if the query fails).
int resident_tiles(int cfg, int device);

hipError_t launch_tile(int cfg, const GemmArgs& a, int device, hipStream_t stream);
hipError_t launch_wsplit(int cfg, const GemmArgs& a, hipStream_t stream);
hipError_t launch_skinny(const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemv(const GemmArgs& a, hipStream_t stream);  // M <= 4

// Grouped (mixture-of-experts) GEMM: G weight operands of N x K, rows of A
// assigned to groups by a device table of G + 1 offsets.
constexpr int kGroupedWaves = 4;   // waves per workgroup (split K)
constexpr int kGroupedChunks = 2;  // 16-row chunks of A per pass over B
constexpr int kGroupedUnits = 1;   // 128-element K units of loads in flight per wave
constexpr int kGroupedBlocks = 4;  // 16-row blocks of B per workgroup (share A's decode)
constexpr int kGroupedTileRows = 464;  // groups this large on average use the tile kernel
constexpr int kGroupedWsplitRows = 33;   // groups this large (and below kGroupedTileRows) on
                                         // average use the grouped mid-size kernel
constexpr int kGroupedWsplitWaves = 8;   // waves per workgroup of that kernel (split K)
constexpr int kGroupedWsplitMaxGroups = 4096;  // its LDS table of row blocks per group

struct GroupedArgs {
    const uint8_t* a_codes;   // [P][Mp][32], all M rows
    const uint8_t* a_scales;  // [P][Mp][4]
    const uint8_t* b_codes;   // G x [P][Np][32]
    const uint8_t* b_scales;  // G x [P][Np][4]
    const int32_t* offsets;   // [G + 1] row offsets (device)
    uint16_t* out;            // [M][N] bfloat16 bits
    float alpha;
    int M, N;                 // total rows of A / C, columns of C
    int Mp, Np;               // padded row counts of the packed operands
    int P;                    // number of 64-element K panels (even)
    int G;                    // number of groups
};
hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream);
hipError_t launch_grouped_wsplit(const GroupedArgs& a, hipStream_t stream);

// Grouped GEMM with large groups on the tile kernel (256 x 256 tiles): one
// workgroup per (row block of a group, column block) of an upper bound of
// tiles_m = ceil(M / 256) + groups row blocks.
hipError_t launch_grouped_tile(const GemmArgs& a, hipStream_t stream);

// Static split-K scratch of the allocation-free entry point
// (nvfp4_gemm_noalloc): arrival counters, then flagged partial words, then
// FP32 partial tiles.
constexpr size_t kScratchCounters = 16384;
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr size_t kScratchFlaggedWords = (size_t)1 << 20;
constexpr size_t kScratchPartialFloats =
    (kScratchBytes - kScratchCounters * 4 - kScratchFlaggedWords * 8) / 4;
// Looks up the device address of the scratch array on `device` (made
// current for the call) once; returns its status.
int noalloc_setup(int device);

// NVFP4 quantisation of fp32 rows into the packed operand layout.
struct QuantArgs {
    const void* x;    // rows x K values (fp32, or bfloat16 if bf16), row stride ld elements
    bool bf16;
    uint8_t* codes;   // packed codes  [P][Rp][32]
    uint8_t* scales;  // packed scales [P][Rp][4]
    int64_t ld;
    int rows, K;
    int Rp, P;        // padded rows, 64-element panels
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);

// The dot-product GEMM with the quantisation of A folded in (M <= 4): A as
// fp32 or bfloat16 rows, quantised per workgroup into LDS.
struct GemvQuantArgs {
    const void* x;    // M x K values (fp32, or bfloat16 if bf16), row stride ldx elements
    bool bf16;
    int64_t ldx;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    uint16_t* out;
    float alpha;
    int M, N, K;
    int Np, P;        // B's padded rows, 64-element panels
};
// Rows of A (rounded up to 1, 2 or 4) x Kp held in LDS at most: 32 KB of
// codes and 4 KB of scales.
constexpr int kGemvQuantElems = 65536;
inline int gemv_rows(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : 4; }
hipError_t launch_gemv_quant(const GemvQuantArgs& a, hipStream_t stream);

}  // namespace nvfp4
