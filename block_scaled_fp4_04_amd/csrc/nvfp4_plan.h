// nvfp4_plan.h -- host-side launch planning of the NVFP4 GEMM (not part of
// the public ABI): the library's rules and the tuned plan table.
#pragma once
#include <stdint.h>

namespace nvfp4 {

struct Plan {
    int path;     // NVFP4_PATH_TILE / _SKINNY / _WSPLIT / _GEMV
    int cfg;      // TileConfig (tile path) or WsplitConfig (wsplit path)
    int split_k;  // number of K slices (>= 1)
    int tiles_m, tiles_n;
    int tail_tiles, tail_split;  // tile path without split-K: last tiles split along K
    int source;   // NVFP4_PLAN_HEURISTIC or NVFP4_PLAN_TABLE
};

// Plan for a shape.  path / tile / split_req as in nvfp4_gemm_with_plan
// (NVFP4_PATH_AUTO with tile 0 and split_req 0 consults the loaded table
// first).  Returns NVFP4_OK, or NVFP4_ERR_INVALID_VALUE for a tile the path
// does not have.  Sizes must already be valid.
int make_plan(int64_t M, int64_t N, int64_t K, int path, int tile, int split_req, Plan* out);

}  // namespace nvfp4
