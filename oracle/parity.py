"""Parity rule of the NVFP4 GEMM and the element sets it is checked on.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the tests, the smoke
check and the CPU leg of the benchmark use it; the product path never does.

Per element, |gpu - oracle| <= ulp_bf16(oracle) + 1e-5 * |alpha| * sum_k |a'_k b'_k|:
one bfloat16 unit in the last place (the GPU rounds its FP32 sum once, the
oracle its exact fp64 sum once) plus a relative allowance for the order of
FP32 additions.  The oracle's sum is exact, and at the benchmark's sizes the
GPU's FP32 sums are exact too, so results are expected to match bit for bit;
the report gives that fraction.
"""
from __future__ import annotations

import time

import numpy as np

from oracle import oracle as orc


def compare(gpu_bits: np.ndarray, oracle_bits: np.ndarray, exact: np.ndarray, mag: np.ndarray,
            alpha: float) -> dict:
    """Per-element bound |gpu - oracle| <= ulp_bf16(oracle) + 1e-5*|alpha|*sum|a'b'|,
    where ulp is taken at the larger of the exact and the rounded oracle value
    (so a result on either side of a power of two gets the wider spacing).
    Returns counts; 'over' must be 0."""
    g = orc.bf16_bits_to_float(np.asarray(gpu_bits, np.uint16).astype(np.uint32) & 0xFFFF)
    o = orc.bf16_bits_to_float(np.asarray(oracle_bits, np.uint16))
    ref = np.maximum(np.abs(exact), np.abs(o))
    tol = orc.bf16_ulp(ref) + 1e-5 * abs(alpha) * mag
    err = np.abs(g - o)
    nan_mismatch = int(np.sum(np.isnan(g) != np.isnan(o)))
    finite = ~np.isnan(g) & ~np.isnan(o)
    over = int(np.sum(err[finite] > tol[finite])) + nan_mismatch
    same = (np.asarray(gpu_bits, np.uint16) == np.asarray(oracle_bits, np.uint16)) | (
        (g == 0) & (o == 0))
    ratio = float(np.max(err[finite] / tol[finite])) if np.any(finite) else 0.0
    return {"n": int(g.size), "over": over, "bit_exact": int(np.sum(same)),
            "bit_exact_frac": float(np.mean(same)) if g.size else 1.0,
            "max_err_over_tol": ratio, "all_zero": bool(np.all(g == 0))}


def merge(reports: list[dict]) -> dict:
    """One report for several disjoint element sets."""
    n = sum(r["n"] for r in reports)
    exact = sum(r["bit_exact"] for r in reports)
    return {"n": n, "over": sum(r["over"] for r in reports), "bit_exact": exact,
            "bit_exact_frac": exact / n if n else 1.0,
            "max_err_over_tol": max((r["max_err_over_tol"] for r in reports), default=0.0),
            "all_zero": all(r["all_zero"] for r in reports)}


# ---------------------------------------------------------------------------
# Element sets for outputs too large to check whole.

def tile_origin(t: int, tiles_m: int, tiles_n: int, tile: int = 256, group_m: int = 8):
    """Output origin (m0, n0) of tile t in the tile order of the persistent
    GEMM launch: tiles are walked in groups of ``group_m`` tile rows, column
    by column inside a group."""
    in_group = group_m * tiles_n
    first_m = (t // in_group) * group_m
    gsize = min(tiles_m - first_m, group_m)
    return (first_m + (t % in_group) % gsize) * tile, ((t % in_group) // gsize) * tile


def large_sample(M: int, N: int, tile: int = 256, xcds: int = 8, random_points: int = 4096,
                 seed: int = 5) -> dict:
    """Elements to check for a large output: four whole rows (0, tile - 1,
    tile, M - 1) and four whole columns (same for N); whole tile x tile
    blocks at the first tile of the grid, the first tile of each XCD's
    contiguous range of tiles (the persistent launch deals tile t to XCD
    t // (T / xcds) when the tile count T is a multiple of xcds), and the
    last tile; and ``random_points`` random elements.
    Returns {"rows": [...], "cols": [...], "tiles": [(m0, n0), ...],
    "points": (ms, ns)}."""
    tiles_m, tiles_n = -(-M // tile), -(-N // tile)
    T = tiles_m * tiles_n
    firsts = [0]
    if T % xcds == 0:
        firsts += [x * (T // xcds) for x in range(1, xcds)]
    firsts.append(T - 1)
    tiles = []
    for t in firsts:
        o = tile_origin(t, tiles_m, tiles_n, tile)
        if o not in tiles:
            tiles.append(o)
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = sorted({0, tile - 1, tile, M - 1} & set(range(M)))
    cols = sorted({0, tile - 1, tile, N - 1} & set(range(N)))
    return {"rows": rows, "cols": cols, "tiles": tiles,
            "points": (rng.integers(0, M, random_points), rng.integers(0, N, random_points))}


def check_sample(o, ops, gpu_bits: np.ndarray, sample: dict, tile: int = 256,
                 col_chunk: int = 2048) -> dict:
    """Compares the GPU output (uint16 bf16 bits, M x N) with the oracle on
    every element of ``sample`` (see large_sample); each part is an ordinary
    oracle GEMM of the rows and columns involved.  Returns the merged report
    plus the number of elements and the oracle's wall time."""
    M, N = gpu_bits.shape
    a_c, a_s, b_c, b_s, alpha = ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha
    reports = []
    t0 = time.perf_counter()
    rows = np.asarray(sample["rows"], np.int64)
    if rows.size:
        bits, ex, mg = o.gemm(np.ascontiguousarray(a_c[rows]), np.ascontiguousarray(a_s[rows]),
                              b_c, b_s, alpha)
        reports.append(compare(gpu_bits[rows], bits, ex, mg, alpha))
    cols = np.asarray(sample["cols"], np.int64)
    if cols.size:
        bc, bs = np.ascontiguousarray(b_c[cols]), np.ascontiguousarray(b_s[cols])
        for r0 in range(0, M, col_chunk):
            r1 = min(M, r0 + col_chunk)
            bits, ex, mg = o.gemm(a_c[r0:r1], a_s[r0:r1], bc, bs, alpha)
            reports.append(compare(gpu_bits[r0:r1][:, cols], bits, ex, mg, alpha))
    for m0, n0 in sample["tiles"]:
        m1, n1 = min(M, m0 + tile), min(N, n0 + tile)
        bits, ex, mg = o.gemm(a_c[m0:m1], a_s[m0:m1], b_c[n0:n1], b_s[n0:n1], alpha)
        reports.append(compare(gpu_bits[m0:m1, n0:n1], bits, ex, mg, alpha))
    ms, ns = sample["points"]
    if len(ms):
        pb, pe, pm = o.gemm_points(a_c, a_s, b_c, b_s, alpha, ms, ns)
        reports.append(compare(gpu_bits[ms, ns], pb, pe, pm, alpha))
    r = merge(reports)
    r["oracle_s"] = time.perf_counter() - t0
    return r
