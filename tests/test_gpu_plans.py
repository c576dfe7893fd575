"""GPU parity of forced launch plans (nvfp4_gemm_with_plan): every tiled
path and tile size with several split-K factors on a ragged shape, and the
persistent tile grid (more tiles than resident workgroups) for each tile
size, against the oracle element by element."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from parity import compare
from plan_cases import TILED, TILED_SPLITS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU hosts, skipped there
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_04_amd as nv  # noqa: E402

DEV = "cuda"


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def o():
    return orc.load()


@pytest.fixture(scope="module")
def ragged(o):
    """300 x 200 x 2192: ragged in M and N for every tile, K not a multiple
    of 128 (zero panels at the end), 18 K steps."""
    ops = synth.random_operands(4242, 300, 200, 2192, alpha=-0.75)
    ref = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    return ops, ref, a, b


@pytest.mark.parametrize("split_k", TILED_SPLITS)
@pytest.mark.parametrize("path,tile", TILED)
def test_forced_plan(ragged, path, tile, split_k):
    ops, (bits, exact, mag), a, b = ragged
    say(f"forced plan {nv.PATH_NAMES[path]} tile {tile} split {split_k}: "
        f"{ops.M}x{ops.N}x{ops.K}")
    out = nv.gemm(a, b, ops.alpha, path=path, tile=tile, split_k=split_k)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    r = compare(g, bits, exact, mag, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r


@pytest.mark.parametrize("split_k", [1, 2, 4, 8])
def test_forced_skinny(o, split_k):
    ops = synth.random_operands(4343, 9, 200, 2192, alpha=0.5)
    say(f"forced skinny split {split_k}: {ops.M}x{ops.N}x{ops.K}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha, path=nv.PATH_SKINNY, split_k=split_k)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(g, bits, exact, mag, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r


@pytest.mark.parametrize("split_k", [1, 3])
@pytest.mark.parametrize("M", [17, 32, 33, 48, 49, 64])
def test_skinny_several_row_blocks(o, M, split_k):
    """The skinny kernel with 2-4 blocks of 16 rows of A sharing each decoded
    B fragment (ragged last block), with and without split-K."""
    ops = synth.random_operands(4444 + M, M, 200, 2192, alpha=-1.5)
    say(f"skinny {M} rows split {split_k}: {ops.M}x{ops.N}x{ops.K}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha, path=nv.PATH_SKINNY, split_k=split_k)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(g, bits, exact, mag, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r


@pytest.mark.parametrize("tile", [256, 128, 64])
def test_persistent_grid_each_tile(o, tile):
    """5100 x 5104 x 576: 400, 1600 and 6400 tiles of 256, 128 and 64, more
    than the workgroups resident on the GPU, so each workgroup walks several
    tiles (N % 8 == 0: the 256 x 256 tiles store through the LDS staging
    block); sampled elements (edge rows and columns, random ones)."""
    M, N = 5100, 5104
    K = 576
    ops = synth.random_operands(977 + tile, M, N, K, alpha=1.5)
    say(f"persistent tile {tile}: {M}x{N}x{K}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha, path=nv.PATH_TILE, tile=tile, split_k=1)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    rng = np.random.Generator(np.random.PCG64(tile))
    edges_m = np.array([0, tile - 1, tile, M - 1 - (M % tile), M - (M % tile), M - 1])
    edges_n = np.array([0, tile - 1, tile, N - 1 - (N % tile), N - (N % tile), N - 1])
    ms = np.concatenate([np.repeat(edges_m, 256), rng.integers(0, M, 2048)])
    ns = np.concatenate([rng.integers(0, N, 256 * len(edges_m)), rng.integers(0, N, 2048)])
    ms = np.concatenate([ms, rng.integers(0, M, 256 * len(edges_n))])
    ns = np.concatenate([ns, np.repeat(edges_n, 256)])
    pb, pe, pm = o.gemm_points(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha,
                               ms, ns)
    r = compare(g[ms, ns], pb, pe, pm, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r
    gf = orc.bf16_bits_to_float(g)
    assert np.all(np.isfinite(gf)) and np.count_nonzero(g & 0x7FFF) > 0.99 * g.size


@pytest.mark.parametrize("M,N,K,tail,split", [(4096, 6144, 512, 128, 2), (4352, 4352, 1024, 33, 4)])
def test_tail_split_launch(o, M, N, K, tail, split):
    """256 x 256 tiles whose last round would be at most half full: the
    full rounds run as one launch and the last tiles as a second launch
    with K split (384 tiles: 128 split 2 ways; 289 tiles: 33 split 4 ways);
    sampled elements all over C, a third of them in the tail's tiles."""
    p = nv.plan(M, N, K)
    assert (p["path"], p["tile_m"], p["split_k"], p["tail_tiles"], p["tail_split"]) == \
        (nv.PATH_TILE, 256, 1, tail, split), p
    ops = synth.random_operands(31 * M + K, M, N, K, alpha=0.875)
    say(f"tail split {tail}x{split}: {M}x{N}x{K}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    rng = np.random.Generator(np.random.PCG64(M + N))
    ms = np.concatenate([rng.integers(0, M, 4096), np.full(256, M - 1), np.arange(256)])
    ns = np.concatenate([rng.integers(0, N, 4096), rng.integers(0, N, 256), np.full(256, N - 1)])
    pb, pe, pm = o.gemm_points(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha,
                               ms, ns)
    r = compare(g[ms, ns], pb, pe, pm, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r
    gf = orc.bf16_bits_to_float(g)
    assert np.all(np.isfinite(gf)) and np.count_nonzero(g & 0x7FFF) > 0.99 * g.size



@pytest.mark.parametrize("M,K", [(5, 6144), (16, 6160), (16, 8192), (32, 6144), (48, 6144), (64, 8192)])
def test_skinny_units_in_flight(o, M, K):
    """The skinny kernel at the K lengths that give each wave 3 or 4 units of
    loads in flight, including units past the end of the range (re-read with
    zero scales: K = 6160 gives 49 units over 16 waves) and two row blocks,
    whose 3 units' worth runs as 4 with one discarded."""
    ops = synth.random_operands(4500 + M + K, M, 72, K, alpha=0.75)
    say(f"skinny units: {ops.M}x{ops.N}x{ops.K}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha, path=nv.PATH_SKINNY, split_k=1)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(g, bits, exact, mag, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r


@pytest.mark.parametrize("M,N,K", [(1, 40, 2048), (2, 56, 4096), (3, 104, 6144), (1, 8, 6160)])
def test_gemv_half_panels_per_lane(o, M, N, K):
    """The dot-product kernel with 1, 2 and 3 half-panels per lane (K up to
    6144), grids that are not a multiple of the 8 XCDs (row remap), and a
    last half-panel shared by a few lanes only (K = 6160)."""
    ops = synth.random_operands(4600 + M + N + K, M, N, K, alpha=-0.5)
    say(f"gemv half-panels: {ops.M}x{ops.N}x{ops.K}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha, path=nv.PATH_GEMV)
    torch.cuda.synchronize()
    g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(g, bits, exact, mag, ops.alpha)
    say(f"  {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r


def test_library_plans_on_random_shapes(o):
    """The library's own plan (table or rules) on 24 seeded random shapes,
    ragged in M, N and K (K a multiple of 16), element by element against
    the oracle: the rules reach the mid-size kernel's tiles, the skinny
    kernel and the dot-product kernel at these sizes."""
    rng = np.random.Generator(np.random.PCG64(77))
    seen = set()
    for i in range(24):
        if i % 3 < 2:
            M = int(rng.choice([rng.integers(1, 5), rng.integers(5, 65), rng.integers(65, 521)]))
            N = int(rng.integers(1, 521))
        else:  # enough rows and columns for the larger tiles
            M = int(rng.integers(200, 1100))
            N = int(rng.integers(500, 2100))
        K = 16 * int(rng.integers(1, 65))
        p = nv.plan(M, N, K)
        seen.add((p["path"], p["tile"]))
        say(f"random shape {i}: {M}x{N}x{K} plan {nv.PATH_NAMES[p['path']]}/{p['tile']}/{p['split_k']}")
        ops = synth.random_operands(5000 + i, M, N, K, alpha=0.625)
        a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
        b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
        out = nv.gemm(a, b, ops.alpha)
        torch.cuda.synchronize()
        g = out.view(torch.int16).cpu().numpy().astype(np.uint16)
        bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
        r = compare(g, bits, exact, mag, ops.alpha)
        say(f"  {r}")
        assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, (M, N, K, p, r)
    say(f"plans reached: {sorted(seen)}")
