"""GPU parity of the grouped (mixture-of-experts) GEMM through the C ABI.

Each group's rows are compared element by element with the oracle's grouped
GEMM (each group an ordinary GEMM with its own weights), with the same bound
as the single GEMM: 1 bf16 ulp + 1e-5 * |alpha| * sum_k |a'_k b'_k|, and the
bit-exact fraction reported.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from parity import compare

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


def random_grouped(seed, sizes, N, K, alpha=1.0):
    """Uniformly random codes (all 16) and random positive scales."""
    g = np.random.Generator(np.random.PCG64(seed))
    G = len(sizes)
    offsets = np.zeros(G + 1, np.int32)
    offsets[1:] = np.cumsum(sizes)
    M = int(offsets[-1])
    ac = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    as_ = g.integers(0x20, 0x49, size=(M, K // 16), dtype=np.uint8)
    bc = g.integers(0, 256, size=(G, N, K // 2), dtype=np.uint8)
    bs = g.integers(0x20, 0x49, size=(G, N, K // 16), dtype=np.uint8)
    return synth.GroupedOperands(ac, as_, bc, bs, offsets, alpha, M, N, K, G)


PATHS = {"auto": nv.PATH_AUTO, "skinny": nv.PATH_SKINNY, "mid": nv.PATH_WSPLIT,
         "tile": nv.PATH_TILE}


def run_grouped(ops, offsets=None, out=None, label="", path="auto"):
    offs = ops.offsets if offsets is None else np.asarray(offsets, np.int32)
    say(f"{label} path={path} G={ops.G} M={ops.M} N={ops.N} K={ops.K} alpha={ops.alpha} "
        f"offsets={offs.tolist() if offs.size <= 12 else '...'}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.groups_to_device(ops.b_codes, ops.b_scales, DEV)
    off = torch.from_numpy(offs).to(DEV)
    c = nv.grouped_gemm(a, b, off, ops.alpha, out=out, path=PATHS[path])
    torch.cuda.synchronize()
    return c.view(torch.int16).cpu().numpy().astype(np.uint16)


def check(o, ops, gpu_bits, label, rows=None):
    bits, exact, mag = o.grouped_gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales,
                                      ops.offsets, ops.alpha)
    sel = slice(None) if rows is None else rows
    r = compare(gpu_bits[sel], bits[sel], exact[sel], mag[sel], ops.alpha)
    say(f"{label}: {r}")
    assert r["over"] == 0, r
    assert r["bit_exact_frac"] >= 0.999, r
    return r


@pytest.mark.parametrize("sizes,N,K", [
    ([0, 1, 16, 17, 40], 40, 640),       # empty group, 1 row, one chunk, two, three (two passes)
    ([3, 0, 0, 33], 16, 128),             # one K step (fewer units than waves)
    ([16] * 9, 256, 6144),                # full K, N of the MoE share
    ([5, 27, 2], 72, 16400),              # K not a multiple of 128 (zero panels)
])
def test_grouped_shapes(o, sizes, N, K):
    ops = random_grouped(sum(sizes) * 7 + N + K, sizes, N, K, alpha=0.75)
    g = run_grouped(ops, label="grouped")
    check(o, ops, g, f"grouped sizes={sizes} N={N} K={K}")


def test_grouped_moe_workload(o):
    """512 tokens routed to 8 of 256 experts (N = 256, K = 6144): the
    benchmark's grouped workload, every element."""
    cfg = synth.grouped_config("moe_up_grouped_e256")
    ops = synth.make_grouped_inputs(cfg)
    g = run_grouped(ops, label="moe grouped workload")
    check(o, ops, g, "moe grouped workload")


def test_grouped_prefill_workload(o):
    """4096 tokens routed to 8 of 256 experts (about 128 rows per expert,
    the mid-size kernel): every element of 16 whole groups (the first, the
    last, the smallest and largest non-empty ones and 12 more at random),
    and every output finite."""
    cfg = synth.grouped_config("moe_up_grouped_e256_t4096")
    ops = synth.make_grouped_inputs(cfg)
    g = run_grouped(ops, label="moe grouped prefill workload")
    counts = np.diff(ops.offsets)
    nonempty = np.flatnonzero(counts)
    rng = np.random.Generator(np.random.PCG64(4096))
    pick = {0, ops.G - 1, int(nonempty[np.argmin(counts[nonempty])]), int(np.argmax(counts))}
    pick |= {int(x) for x in rng.choice(ops.G, size=12, replace=False)}
    say(f"prefill workload: rows per expert {counts.min()}-{counts.max()}, checking groups "
        f"{sorted(pick)}")
    for e in sorted(pick):
        r0, r1 = int(ops.offsets[e]), int(ops.offsets[e + 1])
        if r0 == r1:
            continue
        bits, exact, mag = o.gemm(np.ascontiguousarray(ops.a_codes[r0:r1]),
                                  np.ascontiguousarray(ops.a_scales[r0:r1]), ops.b_codes[e],
                                  ops.b_scales[e], ops.alpha)
        r = compare(g[r0:r1], bits, exact, mag, ops.alpha)
        assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, (e, r)
    vals = orc.bf16_bits_to_float(g)
    assert np.all(np.isfinite(vals))


def test_grouped_offsets_are_clamped_and_rows_outside_groups_untouched(o):
    """A table with entries outside [0, M] is clamped (group 0 empty, group 2
    ends at M); rows after the last group's end are not written."""
    sizes = [4, 3, 7]
    ops = random_grouped(5, sizes, 24, 256, alpha=-1.25)
    M, N = ops.M, ops.N
    # clamped table: [0, -5, 3, 100] acts as [0, 0, 3, M]
    bad = np.array([0, -5, 3, 100], np.int32)
    eff = synth.GroupedOperands(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales,
                                np.array([0, 0, 3, M], np.int32), ops.alpha, M, N, ops.K, 3)
    g = run_grouped(ops, offsets=bad, label="clamped offsets")
    check(o, eff, g, "clamped offsets")
    # last group ends two rows early: those rows keep their previous contents
    short = np.array([0, 4, 7, M - 2], np.int32)
    out = torch.full((M, N), -7.0, dtype=torch.bfloat16, device=DEV)
    g2 = run_grouped(ops, offsets=short, out=out, label="short table")
    eff2 = synth.GroupedOperands(ops.a_codes[:M - 2], ops.a_scales[:M - 2], ops.b_codes,
                                 ops.b_scales, short, ops.alpha, M - 2, N, ops.K, 3)
    check(o, eff2, g2[:M - 2], "short table")
    minus7 = int(torch.tensor([-7.0], dtype=torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    assert np.all(g2[M - 2:] == minus7)


def test_grouped_no_rows():
    """M = 0: nothing to do, success."""
    st = nv.lib().nvfp4_grouped_gemm(0x1000, 0x2000, 0x3000, 0x4000, 0x6000, 4, 1.0, 0x5000,
                                     0, 16, 128, None)
    assert st == nv.OK


# Large groups on the tile kernel (256 x 256 tiles: row blocks of each
# group, with a partial block at every group's end), forced, and each case
# also on the library's choice (the mid-size kernel up to 463 rows on
# average, the tile kernel from 464: the last case) and on the skinny kernel
# (several passes over B per workgroup).
@pytest.mark.parametrize("sizes,N,K", [
    ([0, 70, 130, 1, 257, 64, 200], 200, 640),      # empty and 1-row groups
    ([300, 512, 0, 700, 259], 264, 1040),            # K not a multiple of 128
    ([256] * 4 + [512], 256, 2048),                  # whole 256-row blocks only
    ([1, 1000, 3, 300], 136, 384),                   # tiny and large groups
    ([520, 0, 900, 500], 72, 256),                   # 480 rows on average: tile by default
])
def test_grouped_tile_path(o, sizes, N, K):
    ops = random_grouped(sum(sizes) * 3 + N + K, sizes, N, K, alpha=-0.625)
    for path in ("tile", "auto", "skinny"):
        g = run_grouped(ops, label=f"grouped ({path} path)", path=path)
        check(o, ops, g, f"grouped {path} path sizes={sizes} N={N} K={K}")


# Groups of 33-463 rows on average run on the mid-size kernel: 64 x 64 tiles
# of every group (row blocks from each group's first row, the last one cut
# at the group's end), taken in turn by a persistent grid of at most one
# workgroup per CU.
@pytest.mark.parametrize("sizes,N,K", [
    ([64] * 8, 256, 6144),                            # whole row blocks, full K
    ([65, 63, 128, 129, 0, 191], 136, 1040),          # partial blocks, K not a multiple of 128
    ([96] * 300, 128, 128),                           # 1200 tiles: about 5 per workgroup
    ([0, 1, 2, 500, 3, 0, 64], 40, 256),              # one large group among tiny ones
])
def test_grouped_mid_path(o, sizes, N, K):
    ops = random_grouped(sum(sizes) * 5 + N + K, sizes, N, K, alpha=1.375)
    g = run_grouped(ops, label="grouped (mid-size path)", path="mid")
    check(o, ops, g, f"grouped mid-size path sizes={sizes} N={N} K={K}")


def test_grouped_mid_path_table_limit(o):
    """4096 groups (the mid-size kernel's LDS table holds that many) of 0-5
    rows, forced onto the mid-size kernel: every thread of the prefix sum
    counts eight groups."""
    g = np.random.Generator(np.random.PCG64(4096))
    sizes = [int(s) for s in g.integers(0, 6, size=4096)]
    ops = random_grouped(4097, sizes, 40, 64, alpha=0.5)
    out = run_grouped(ops, label="grouped (mid-size path, 4096 groups)", path="mid")
    check(o, ops, out, "mid-size path, 4096 groups")


def test_grouped_paths_agree(o):
    """The same call on each of the three kernels: every one matches the
    oracle, and all give the same bits.  Scales are 0.5, 1 or 2 (E4M3 bytes
    0x30, 0x38, 0x40), so every product is a multiple of 1/16 of magnitude at
    most 144 and every sum over K = 768 is exact in FP32 (below 2^24 / 16),
    whatever the order of the additions."""
    sizes = [40, 0, 200, 64, 1, 300, 128]
    ops = random_grouped(91, sizes, 160, 768, alpha=-2.0)
    g = np.random.Generator(np.random.PCG64(92))
    pick = np.array([0x30, 0x38, 0x40], np.uint8)
    ops = dataclasses.replace(ops, a_scales=pick[g.integers(0, 3, size=ops.a_scales.shape)],
                              b_scales=pick[g.integers(0, 3, size=ops.b_scales.shape)])
    outs = {}
    for path in ("skinny", "mid", "tile"):
        outs[path] = run_grouped(ops, label=f"grouped ({path} path)", path=path)
        check(o, ops, outs[path], f"grouped {path} path")
    assert np.array_equal(outs["skinny"], outs["mid"])
    assert np.array_equal(outs["skinny"], outs["tile"])


@pytest.mark.parametrize("path", ["tile", "mid"])
def test_grouped_tile_path_clamps_and_leaves_other_rows(o, path):
    """Tile and mid-size paths with a malformed table (entries outside
    [0, M] are clamped) and a table that ends before M (the rows after it
    keep their contents)."""
    sizes = [400, 260, 300]
    ops = random_grouped(77, sizes, 136, 512, alpha=1.5)
    M, N = ops.M, ops.N
    bad = np.array([0, -9, 400, 10 ** 6], np.int32)           # acts as [0, 0, 400, M]
    eff = synth.GroupedOperands(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales,
                                np.array([0, 0, 400, M], np.int32), ops.alpha, M, N, ops.K, 3)
    g = run_grouped(ops, offsets=bad, label=f"{path} path, clamped offsets", path=path)
    check(o, eff, g, f"{path} path, clamped offsets")
    short = np.array([0, 400, 660, M - 70], np.int32)
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    g2 = run_grouped(ops, offsets=short, out=out, label=f"{path} path, short table", path=path)
    eff2 = synth.GroupedOperands(ops.a_codes[:M - 70], ops.a_scales[:M - 70], ops.b_codes,
                                 ops.b_scales, short, ops.alpha, M - 70, N, ops.K, 3)
    check(o, eff2, g2[:M - 70], f"{path} path, short table")
    three = int(torch.tensor([3.0], dtype=torch.bfloat16).view(torch.int16).item()) & 0xFFFF
    assert np.all(g2[M - 70:] == three)
