"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every comparison is element by element on the same seeded inputs.  The
bound is |gpu - oracle| <= 1 bf16 ulp + 1e-5 * |alpha| * sum_k |a'_k b'_k|;
because the kernels decode exactly and accumulate exact products in FP32,
the results are also expected to be bit-identical to the oracle on (almost)
every element, and the tests report that fraction.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth
from oracle import oracle as orc
from parity import check_sample, compare, large_sample, merge

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


def run_gpu(ops: synth.Operands, path=nv.PATH_AUTO, split_k=0, stream=None, label="", tile=0):
    say(f"{label} M={ops.M} N={ops.N} K={ops.K} alpha={ops.alpha} path={path} split_k={split_k} "
        f"tile={tile}")
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    out = nv.gemm(a, b, ops.alpha, path=path, split_k=split_k, stream=stream, tile=tile)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().astype(np.uint16)


def check_full(o, ops, gpu_bits, label, min_exact=0.999):
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(gpu_bits, bits, exact, mag, ops.alpha)
    say(f"{label}: {r}")
    assert r["over"] == 0, r
    assert r["bit_exact_frac"] >= min_exact, r
    return r


# ------------------------------------------------------------ decode and layout

@pytest.mark.parametrize("path", [nv.PATH_TILE, nv.PATH_WSPLIT, nv.PATH_SKINNY, nv.PATH_GEMV])
def test_decode_exhaustive(o, path):
    """Every E4M3 scale byte times every E2M1 code, through the GEMM: one
    operand has a single 1.0 at k=0 with scale s in row s, the other has code
    c at k=0 with scale 1.0 in row c, so C holds every product exactly."""
    K = 64
    sc_rows = np.zeros((256, K // 2), np.uint8)
    sc_rows[:, 0] = 0x02                                   # code 1.0 at k = 0
    sc_scales = np.full((256, K // 16), 0x38, np.uint8)
    sc_scales[:, 0] = np.arange(256, dtype=np.uint8)       # scale byte s in row s
    cd_rows = np.zeros((16, K // 2), np.uint8)
    cd_rows[:, 0] = np.arange(16, dtype=np.uint8)          # code c at k = 0 in row c
    cd_scales = np.full((16, K // 16), 0x38, np.uint8)
    if path == nv.PATH_GEMV:   # M <= 4: four code rows at a time as A
        for c0 in range(0, 16, 4):
            ops = synth.Operands(cd_rows[c0:c0 + 4].copy(), cd_scales[c0:c0 + 4].copy(), sc_rows,
                                 sc_scales, 1.0, 4, 256, K)
            g = run_gpu(ops, path=path, label=f"decode codes {c0}..{c0 + 3}")
            bits, _, _ = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, 1.0)
            nan_o = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
            nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
            assert np.array_equal(nan_o, nan_g)
            ok = ~nan_o
            same = (g[ok] == bits[ok]) | (((g[ok] & 0x7FFF) == 0) & ((bits[ok] & 0x7FFF) == 0))
            assert np.all(same), np.argwhere(~same)[:10]
        return
    if path != nv.PATH_SKINNY:
        ops = synth.Operands(sc_rows, sc_scales, cd_rows, cd_scales, 1.0, 256, 16, K)
    else:   # skinny: M <= 16, so the code rows are A
        ops = synth.Operands(cd_rows, cd_scales, sc_rows, sc_scales, 1.0, 16, 256, K)
    g = run_gpu(ops, path=path, label="decode")
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, 1.0)
    nan_o = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
    nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    assert np.array_equal(nan_o, nan_g)
    ok = ~nan_o
    same = (g[ok] == bits[ok]) | (((g[ok] & 0x7FFF) == 0) & ((bits[ok] & 0x7FFF) == 0))
    assert np.all(same), np.argwhere(~same)[:10]


@pytest.mark.parametrize("path", [nv.PATH_TILE, nv.PATH_WSPLIT, nv.PATH_SKINNY, nv.PATH_GEMV])
def test_onehot_positions(o, path):
    """One non-zero product at a time, at positions across tile, panel and
    scale-block boundaries: pins nibble order, K slots, scale blocks, the
    packer and the MFMA operand/result layouts."""
    M = {nv.PATH_SKINNY: 16, nv.PATH_GEMV: 4}.get(path, 300)
    N, K = 290, 320
    g = np.random.Generator(np.random.PCG64(77))
    for t in range(6):
        m, n, k = int(g.integers(M)), int(g.integers(N)), int(g.integers(K))
        if t == 0:
            m, n, k = M - 1, N - 1, K - 1
        ac = np.zeros((M, K // 2), np.uint8)
        bc = np.zeros((N, K // 2), np.uint8)
        ac[m, k // 2] = 0x5 << (4 * (k % 2))          # 3.0
        bc[n, k // 2] = 0xB << (4 * (k % 2))          # -1.5
        as_ = np.full((M, K // 16), 0x38, np.uint8)
        bs = np.full((N, K // 16), 0x38, np.uint8)
        as_[m, k // 16] = 0x3B                        # 1.375
        bs[n, k // 16] = 0x06                         # subnormal 6 * 2^-9
        ops = synth.Operands(ac, as_, bc, bs, 1.0, M, N, K)
        gb = run_gpu(ops, path=path, label=f"onehot m={m} n={n} k={k}")
        want = np.zeros((M, N), np.uint16)
        bits, _, _ = o.gemm(ac, as_, bc, bs, 1.0)
        assert bits[m, n] != 0 and int(np.count_nonzero(bits & 0x7FFF)) == 1
        nz = np.argwhere(gb & 0x7FFF)
        assert nz.tolist() == [[m, n]], (m, n, k, nz[:5])
        assert gb[m, n] == bits[m, n]
        del want


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_parity_workload(o, i):
    cfg = synth.config(i)
    ops = synth.make_inputs(cfg)
    g = run_gpu(ops, label=f"workload {i} {cfg.name}")
    r = check_full(o, ops, g, f"workload {i}")
    assert not r["all_zero"]


def test_parity_saturation(o):
    """16384 x 8192 x 8192 in the launch configuration the benchmark times
    (persistent 256 x 256 tiles, no split), checked element by element
    against the oracle on: four whole rows and four whole columns (the
    first, both sides of the first tile edge, the last); whole 256 x 256
    tiles at the start of the grid, at the start of each XCD's contiguous
    range of tiles and at the end of the grid; and 4096 random elements.
    Every other element is checked to be finite."""
    import os
    cfg = synth.config(5)
    p = nv.plan(cfg.M, cfg.N, cfg.K)
    assert (p["path"], p["tile_m"], p["split_k"], p["tail_tiles"]) == (nv.PATH_TILE, 256, 1, 0), p
    ops = synth.make_inputs(cfg)
    g = run_gpu(ops, label="workload 5 saturation")
    sample = large_sample(cfg.M, cfg.N)
    assert len(sample["tiles"]) == 9, sample["tiles"]   # 2048 tiles: 8 XCD ranges + the last
    r = check_sample(o, ops, g, sample)
    say(f"workload 5: rows {sample['rows']} cols {sample['cols']} tiles {sample['tiles']} "
        f"+ {len(sample['points'][0])} random: {r} (oracle on {o.threads} threads, "
        f"nproc {os.cpu_count()})")
    assert r["n"] == 4 * cfg.N + 4 * cfg.M + 9 * 256 * 256 + 4096
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r
    gf = orc.bf16_bits_to_float(g)
    assert np.all(np.isfinite(gf)) and np.count_nonzero(g & 0x7FFF) > 0.99 * g.size


# ------------------------------------------------------------ edges

EDGE_SHAPES = [(1, 1, 16), (1, 17, 32), (2, 33, 48), (15, 16, 80), (16, 255, 6160),
               (17, 16, 16), (63, 65, 208), (64, 64, 64), (65, 31, 128), (257, 130, 336),
               (300, 513, 1040)]


@pytest.mark.parametrize("M,N,K", EDGE_SHAPES)
def test_edge_shapes(o, M, N, K):
    """Every path on outputs smaller than one tile and ragged in both
    dimensions, each tile of the mid-size kernel forced (32 x 32, 64 x 32,
    64 x 64, 128 x 64)."""
    ops = synth.random_operands(1000 * M + N + K, M, N, K, alpha=0.75)
    plans = [(nv.PATH_AUTO, 0), (nv.PATH_TILE, 0)] + [(nv.PATH_WSPLIT, t) for t in (16, 32, 64, 128)] \
        + ([(nv.PATH_SKINNY, 0)] if M <= 16 else []) + ([(nv.PATH_GEMV, 0)] if M <= 4 else [])
    for path, tile in plans:
        g = run_gpu(ops, path=path, tile=tile, label="edge")
        check_full(o, ops, g, f"edge {M}x{N}x{K} path {path} tile {tile}")


@pytest.mark.parametrize("M,N,K", [(4100, 4198, 128), (4352, 4096, 640)])
def test_tile_several_tiles_per_workgroup(o, M, N, K):
    """More 256 x 256 tiles than workgroups resident on the GPU, so each
    workgroup walks two tiles with its load ring running across them (with
    K = 128 the look-ahead spans several tiles); ragged edge tiles, both
    output store forms (N % 4 != 0 and N % 4 == 0), and tile counts with and
    without the XCD remap (289 and 272 tiles)."""
    p = nv.plan(M, N, K)
    assert p["path"] == nv.PATH_TILE and p["split_k"] == 1 and p["tile_m"] == 256, p
    ops = synth.random_operands(7 * M + N + K, M, N, K, alpha=0.625)
    g = run_gpu(ops, label="several tiles per workgroup")
    check_full(o, ops, g, f"tile {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (17, 16, 16), (65, 31, 128), (257, 130, 336),
                                   (300, 513, 1040), (520, 264, 4096), (512, 1030, 256)])
def test_tile256_unsplit(o, M, N, K):
    """The unsplit 256 x 256 kernel on its own: outputs smaller than one
    tile, ragged edges in both dimensions (the 128-row quarters that each
    wave decodes reach past the padded rows), N % 8 != 0 and N % 4 != 0
    (the direct stores) beside N % 8 == 0 (the staged ones), and K from one
    panel pair up to 64 panels."""
    ops = synth.random_operands(31 * M + 7 * N + K, M, N, K, alpha=-1.5)
    g = run_gpu(ops, path=nv.PATH_TILE, tile=256, split_k=1, label="tile 256 unsplit")
    check_full(o, ops, g, f"tile 256 {M}x{N}x{K}")


@pytest.mark.parametrize("big", ["a", "b"])
def test_operand_just_under_32bit_offsets(o, big):
    """One operand one row block under the tile and wsplit kernels' 32-bit
    byte-offset limit (packed codes 2048 panels x 32752 rows x 32 bytes =
    2 GiB - 1 MiB), the other 512 rows, K = 131072: the library's plan and
    every forced tile and wsplit plan against the oracle on the last 2048
    elements of the last row and of the last column (each reads the highest
    panels; together they take the highest rows of both operands) and 2048
    random elements, one oracle pass for all."""
    K = 131072
    M, N = (32752, 512) if big == "a" else (512, 32752)
    say(f"generating {M}x{N}x{K} operands")
    ops = synth.random_operands(4242 + M, M, N, K, alpha=0.5)
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    m0, n0 = max(0, M - 2048), max(0, N - 2048)
    ms = np.random.Generator(np.random.PCG64(9)).integers(0, M, 2048)
    ns = np.random.Generator(np.random.PCG64(10)).integers(0, N, 2048)
    outs = {}
    for path, tile in ((nv.PATH_AUTO, 0), (nv.PATH_TILE, 256), (nv.PATH_TILE, 128),
                       (nv.PATH_WSPLIT, 16), (nv.PATH_WSPLIT, 32), (nv.PATH_WSPLIT, 64),
                       (nv.PATH_WSPLIT, 128)):
        say(f"{big}: path {path} tile {tile}")
        g = nv.gemm(a, b, ops.alpha, path=path, tile=tile)
        torch.cuda.synchronize()
        outs[(path, tile)] = g.view(torch.int16).cpu().numpy().astype(np.uint16)
        del g
    del a, b
    # the oracle's values of the sampled elements, computed once
    row = o.gemm(np.ascontiguousarray(ops.a_codes[M - 1:]), np.ascontiguousarray(ops.a_scales[M - 1:]),
                 np.ascontiguousarray(ops.b_codes[n0:]), np.ascontiguousarray(ops.b_scales[n0:]),
                 ops.alpha)
    col = o.gemm(np.ascontiguousarray(ops.a_codes[m0:]), np.ascontiguousarray(ops.a_scales[m0:]),
                 np.ascontiguousarray(ops.b_codes[N - 1:]), np.ascontiguousarray(ops.b_scales[N - 1:]),
                 ops.alpha)
    pts = o.gemm_points(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha, ms, ns)
    for key, g in outs.items():
        r = merge([compare(g[M - 1:, n0:], *row, ops.alpha), compare(g[m0:, N - 1:], *col, ops.alpha),
                   compare(g[ms, ns], *pts, ops.alpha)])
        say(f"{big} {key}: {r}")
        assert r["over"] == 0 and r["bit_exact_frac"] >= 0.99 and not r["all_zero"], (key, r)


@pytest.mark.parametrize("alpha", [0.0, -0.0, -1.75, 1e36, -1e36, 1e-40, 3e-39,
                                   float("inf"), float("-inf"), float("nan")])
def test_alpha_special_values(o, alpha):
    """The epilogue's degenerate cases on every path: alpha of either zero,
    products past the bfloat16 range (1e36 x sums of a few hundred or more),
    results among the bfloat16 subnormals (alpha 1e-40 and 3e-39, both FP32
    subnormals themselves: a flushed denormal would show as zeros), infinite
    alpha (sums of zero give NaN) and NaN.  NaN positions must match the oracle's and
    every other element its bits (zeros of either sign count as equal),
    infinities included: with an infinite alpha the relative tolerance says
    nothing."""
    for M, paths in ((40, (nv.PATH_AUTO, nv.PATH_TILE, nv.PATH_WSPLIT, nv.PATH_SKINNY)),
                     (3, (nv.PATH_AUTO, nv.PATH_GEMV))):
        ops = synth.random_operands(77 + M, M, 72, 256, alpha=alpha)
        bits, _, _ = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, alpha)
        nan_o = ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
        for path in paths:
            g = run_gpu(ops, path=path, label=f"alpha {alpha}")
            nan_g = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
            ok = ~nan_o
            same = (g[ok] == bits[ok]) | (((g[ok] & 0x7FFF) == 0) & ((bits[ok] & 0x7FFF) == 0))
            say(f"alpha {alpha} M {M} path {path}: NaN {int(nan_o.sum())}/{int(nan_g.sum())}, "
                f"bit-equal {float(same.mean()) if same.size else 1.0}")
            assert np.array_equal(nan_o, nan_g), (alpha, path)
            assert same.all(), (alpha, path, g[ok][~same][:8], bits[ok][~same][:8])


@pytest.mark.parametrize("split_k", [1, 2, 3, 5, 16])
def test_split_k_variants(o, split_k):
    ops = synth.quantized_operands(91, 200, 160, 2048, alpha=1.25)
    g = run_gpu(ops, path=nv.PATH_TILE, split_k=split_k, label="split-k tile")
    check_full(o, ops, g, f"tile split {split_k}")
    g = run_gpu(ops, path=nv.PATH_WSPLIT, split_k=split_k, label="split-k wsplit")
    check_full(o, ops, g, f"wsplit split {split_k}")
    ops16 = synth.quantized_operands(92, 9, 300, 2048, alpha=-0.5)
    g = run_gpu(ops16, path=nv.PATH_SKINNY, split_k=split_k, label="split-k skinny")
    check_full(o, ops16, g, f"skinny split {split_k}")


@pytest.mark.parametrize("M,K", [(1, 16), (2, 8320), (3, 16400), (4, 24576)])
def test_gemv_k_chunks(o, M, K):
    """The dot-product path over K longer than one 8192-element chunk."""
    ops = synth.quantized_operands(93 + M, M, 72, K, alpha=0.25)
    g = run_gpu(ops, path=nv.PATH_GEMV, label="gemv chunks")
    check_full(o, ops, g, f"gemv {M}x72x{K}")


def test_wide_scale_range(o):
    """Scale bytes across the whole finite range (negative, subnormal, 448)."""
    g0 = np.random.Generator(np.random.PCG64(123))
    M, N, K = 96, 80, 256
    fin = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    ops = synth.Operands(g0.integers(0, 256, (M, K // 2), dtype=np.uint8),
                         g0.choice(fin, (M, K // 16)).astype(np.uint8),
                         g0.integers(0, 256, (N, K // 2), dtype=np.uint8),
                         g0.choice(fin, (N, K // 16)).astype(np.uint8), 1.0, M, N, K)
    for path, tile in ((nv.PATH_TILE, 0), (nv.PATH_TILE, 256), (nv.PATH_WSPLIT, 0)):
        g = run_gpu(ops, path=path, tile=tile, label="wide scales")
        check_full(o, ops, g, "wide scales", min_exact=0.99)


# ------------------------------------------------------------ properties

def test_determinism_and_symmetry(o):
    ops = synth.quantized_operands(5, 64, 96, 1024)
    g1 = run_gpu(ops, split_k=4, path=nv.PATH_TILE, label="determinism 1")
    g2 = run_gpu(ops, split_k=4, path=nv.PATH_TILE, label="determinism 2")
    assert np.array_equal(g1, g2)
    w1 = run_gpu(ops, split_k=3, path=nv.PATH_WSPLIT, label="determinism wsplit 1")
    w2 = run_gpu(ops, split_k=3, path=nv.PATH_WSPLIT, label="determinism wsplit 2")
    assert np.array_equal(w1, w2) and np.array_equal(w1, g1)
    t = synth.Operands(ops.b_codes, ops.b_scales, ops.a_codes, ops.a_scales, 1.0, 96, 64, 1024)
    gt = run_gpu(t, path=nv.PATH_TILE, label="transpose")
    assert np.array_equal(gt, g1.T)
    s1 = synth.make_inputs(synth.config(1))
    a1 = run_gpu(s1, label="determinism skinny 1")
    a2 = run_gpu(s1, label="determinism skinny 2")
    assert np.array_equal(a1, a2)


def test_out_guard_and_stream(o):
    """The kernels write exactly M x N elements (guard words around the
    output stay intact) and run on a caller's stream."""
    ops = synth.random_operands(8, 33, 70, 192)
    a = nv.to_device(ops.a_codes, ops.a_scales, DEV)
    b = nv.to_device(ops.b_codes, ops.b_scales, DEV)
    for path in (nv.PATH_TILE, nv.PATH_SKINNY) if ops.M <= 16 else (nv.PATH_TILE, nv.PATH_WSPLIT):
        say(f"guard path={path}")
        buf = torch.full((33 * 70 + 2 * 64,), -12345, dtype=torch.int16, device=DEV)
        out = buf[64:64 + 33 * 70].view(torch.bfloat16).view(33, 70)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            nv.gemm(a, b, 1.0, out=out, path=path, stream=s)
        s.synchronize()
        host = buf.cpu().numpy()
        assert np.all(host[:64] == -12345) and np.all(host[64 + 33 * 70:] == -12345)
        g = host[64:64 + 33 * 70].astype(np.uint16).reshape(33, 70)
        check_full(o, ops, g, "guard")
