"""Launch plans (path, tile, split-K) that the GPU parity tests force, so the
tuned table can be checked to choose only among them."""
import block_scaled_fp4_04_amd as nv

TILED = [(nv.PATH_TILE, 256), (nv.PATH_TILE, 128), (nv.PATH_TILE, 64), (nv.PATH_WSPLIT, 16),
         (nv.PATH_WSPLIT, 32), (nv.PATH_WSPLIT, 64), (nv.PATH_WSPLIT, 128)]
TILED_SPLITS = [1, 2, 3, 4, 6, 8]
SKINNY_SPLITS = [1, 2, 3, 4, 5, 8, 16]   # forced in the split-K and forced-plan tests


def tested(path_name: str, tile: int, split_k: int) -> bool:
    path = {v: k for k, v in nv.PATH_NAMES.items()}[path_name]
    if path == nv.PATH_GEMV:
        return split_k == 1
    if path == nv.PATH_SKINNY:
        return split_k in SKINNY_SPLITS
    if tile == 0:  # the path's own choice: one of its tiles, all of them forced
        return any(p == path for p, _ in TILED) and split_k in TILED_SPLITS
    return (path, tile) in TILED and split_k in TILED_SPLITS
