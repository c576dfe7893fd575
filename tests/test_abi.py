"""The C-ABI library: symbols, host-side packing and argument validation.

No GPU is needed: every check here happens on the host before any launch
(nvfp4_gemm validates its arguments before touching the device)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_scaled_fp4_04_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(nvfp4_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = nv.lib()
    declared = header_functions()
    assert len(declared) >= 10, declared
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/nvfp4.h but not exported"
    assert sorted(nv.EXPORTS) == declared


def test_status_strings():
    names = {nv.status_string(st) for st in range(8)}
    assert len(names) == 8 and "unknown status" not in names
    assert nv.status_string(99) == "unknown status"
    assert nv.version() >= 100


@pytest.mark.parametrize("rows,K", [(1, 16), (15, 48), (16, 64), (17, 6144), (256, 8192),
                                    (1000, 6160)])
def test_packed_size(rows, K):
    cb, sb = nv.packed_size(rows, K)
    Rp = -(-rows // 16) * 16
    Kp = -(-K // 128) * 128
    assert cb == Rp * Kp // 2 and sb == Rp * Kp // 16


@pytest.mark.parametrize("rows,K", [(0, 64), (4, 0), (4, 24), (4, -16), (-1, 64)])
def test_packed_size_rejects(rows, K):
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.packed_size(rows, K)
    assert e.value.status == nv.ERR_INVALID_VALUE


@pytest.mark.parametrize("rows,K", [(1, 16), (5, 48), (16, 64), (33, 208), (100, 6144)])
def test_pack_roundtrip_and_layout(rows, K):
    g = np.random.default_rng(rows * 1000 + K)
    codes = g.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    scales = g.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    pc, ps = nv.pack(codes, scales)
    c2, s2 = nv.unpack(pc, ps, rows, K)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # layout: panel p, row r holds canonical bytes [32p, 32p+32) and scales [4p, 4p+4)
    Rp, P = -(-rows // 16) * 16, 2 * -(-K // 128)
    pc3 = pc.reshape(P, Rp, 32)
    ps3 = ps.reshape(P, Rp, 4)
    for p in range(P):
        n = max(0, min(32, K // 2 - 32 * p))
        assert np.array_equal(pc3[p, :rows, :n], codes[:, 32 * p:32 * p + n])
        assert not pc3[p, :rows, n:].any() and not pc3[p, rows:].any()
        ns = max(0, min(4, K // 16 - 4 * p))
        assert np.array_equal(ps3[p, :rows, :ns], scales[:, 4 * p:4 * p + ns])
        assert not ps3[p, :rows, ns:].any() and not ps3[p, rows:].any()


def test_pack_rejects_bad_shapes():
    with pytest.raises(ValueError):
        nv.pack(np.zeros((2, 8), np.uint8), np.zeros((2, 2), np.uint8))
    with pytest.raises(ValueError):
        nv.pack(np.zeros((2, 12), np.uint8), np.zeros((2, 1), np.uint8))   # K = 24


def _raw(a=0x1000, sa=0x2000, b=0x3000, sb=0x4000, out=0x5000, M=4, N=4, K=64):
    lib = nv.lib()
    return lib.nvfp4_gemm(a, sa, b, sb, 1.0, out, M, N, K, None)


def test_gemm_rejects_bad_arguments_before_launch():
    assert _raw(a=None) == nv.ERR_INVALID_VALUE
    assert _raw(out=None) == nv.ERR_INVALID_VALUE
    assert _raw(M=0) == nv.ERR_INVALID_VALUE
    assert _raw(N=-3) == nv.ERR_INVALID_VALUE
    assert _raw(K=0) == nv.ERR_INVALID_VALUE
    assert _raw(K=24) == nv.ERR_INVALID_VALUE    # K not a multiple of the block size
    assert _raw(K=8) == nv.ERR_INVALID_VALUE
    assert _raw(a=0x1004) == nv.ERR_MISALIGNED
    assert _raw(out=0x5002) == nv.ERR_MISALIGNED
    lib = nv.lib()
    # a forced skinny path needs M <= 64
    assert _wp(65, 4, 64, nv.PATH_SKINNY) == nv.ERR_UNSUPPORTED
    assert _wp(5, 4, 64, nv.PATH_GEMV) == nv.ERR_UNSUPPORTED
    assert _wp(4, 4, 64, 7) == nv.ERR_INVALID_VALUE
    assert _wp(4, 4, 64, 0, split_k=-1) == nv.ERR_INVALID_VALUE
    # tiles the path does not have
    for path, tile in [(nv.PATH_AUTO, 128), (nv.PATH_TILE, 96), (nv.PATH_TILE, 32),
                       (nv.PATH_WSPLIT, 256), (nv.PATH_WSPLIT, 48), (nv.PATH_WSPLIT, 8),
                       (nv.PATH_SKINNY, 16), (nv.PATH_GEMV, 4), (nv.PATH_TILE, -1)]:
        assert _wp(4, 32, 64, path, tile) == nv.ERR_INVALID_VALUE, (path, tile)


def test_gemm_refuses_operands_past_32bit_offsets():
    """The tile and wsplit kernels address a packed operand with 32-bit byte
    offsets, so a tile or wsplit plan whose packed codes would reach 2 GiB
    (32768 rows x 131072 K: 2048 panels x 32768 rows x 32 bytes) is refused
    before launch, for A and for B, forced or chosen by the library.  (Only
    refusals are asserted here: an accepted call would launch on a GPU host;
    the GPU parity tests run operands one row-block under the limit.)"""
    K = 131072
    for path, tile in ((nv.PATH_TILE, 256), (nv.PATH_TILE, 128), (nv.PATH_WSPLIT, 16),
                       (nv.PATH_WSPLIT, 32), (nv.PATH_WSPLIT, 64), (nv.PATH_WSPLIT, 128),
                       (nv.PATH_AUTO, 0)):
        assert _wp(32768, 256, K, path, tile) == nv.ERR_UNSUPPORTED, (path, tile)
        assert _wp(256, 32768, K, path, tile) == nv.ERR_UNSUPPORTED, (path, tile)


def _wp(M, N, K, path, tile=0, split_k=0):
    return nv.lib().nvfp4_gemm_with_plan(0x1000, 0x2000, 0x3000, 0x4000, 1.0, 0x5000, M, N, K,
                                         path, tile, split_k, None)


def _graw(a=0x1000, sa=0x2000, b=0x3000, sb=0x4000, off=0x6000, G=4, out=0x5000, M=4, N=4,
          K=64):
    return nv.lib().nvfp4_grouped_gemm(a, sa, b, sb, off, G, 1.0, out, M, N, K, None)


def test_grouped_gemm_rejects_bad_arguments_before_launch():
    assert _graw(a=None) == nv.ERR_INVALID_VALUE
    assert _graw(off=None) == nv.ERR_INVALID_VALUE
    assert _graw(out=None) == nv.ERR_INVALID_VALUE
    assert _graw(G=0) == nv.ERR_INVALID_VALUE
    assert _graw(M=-1) == nv.ERR_INVALID_VALUE
    assert _graw(N=0) == nv.ERR_INVALID_VALUE
    assert _graw(K=24) == nv.ERR_INVALID_VALUE
    assert _graw(G=1 << 30, N=256) == nv.ERR_INVALID_VALUE   # grid too large
    assert _graw(b=0x3008) == nv.ERR_MISALIGNED
    assert _graw(off=0x6002) == nv.ERR_MISALIGNED


def _gwp(path, G=4, M=4, N=4, K=64, b=0x3000):
    return nv.lib().nvfp4_grouped_gemm_with_plan(0x1000, 0x2000, b, 0x4000, 0x6000, G, 1.0,
                                                 0x5000, M, N, K, path, None)


def test_grouped_gemm_with_plan_rejects_bad_paths_and_sizes_before_launch():
    # only the three grouped kernels (or the library's choice) can be forced
    for path in (-1, nv.PATH_GEMV, 5, 99):
        assert _gwp(path) == nv.ERR_INVALID_VALUE, path
    # the checks of nvfp4_grouped_gemm come first, for every path
    for path in (nv.PATH_AUTO, nv.PATH_SKINNY, nv.PATH_WSPLIT, nv.PATH_TILE):
        assert _gwp(path, G=0) == nv.ERR_INVALID_VALUE, path
        assert _gwp(path, K=24) == nv.ERR_INVALID_VALUE, path
        assert _gwp(path, b=0x3008) == nv.ERR_MISALIGNED, path
    # the mid-size kernel's LDS table holds at most 4096 groups
    assert _gwp(nv.PATH_WSPLIT, G=4097, M=4097 * 64) == nv.ERR_UNSUPPORTED
    # the mid-size and tile kernels address A (and each group's B) with
    # 32-bit offsets: 2 GiB of packed codes or more cannot be forced there,
    # while the skinny kernel and the library's choice (which falls back to
    # it) take them
    big_m = (1 << 31) // (6144 // 2) + 16   # rows of K = 6144 past 2 GiB of codes
    for path in (nv.PATH_WSPLIT, nv.PATH_TILE):
        assert _gwp(path, G=4, M=big_m, N=256, K=6144) == nv.ERR_UNSUPPORTED, path


def test_pack_groups_concatenates_per_group_packing():
    g = np.random.Generator(np.random.PCG64(3))
    codes = g.integers(0, 256, size=(3, 20, 80), dtype=np.uint8)
    scales = g.integers(0, 256, size=(3, 20, 10), dtype=np.uint8)
    pc, ps = nv.pack_groups(codes, scales)
    cb, sb = nv.packed_size(20, 160)
    assert pc.size == 3 * cb and ps.size == 3 * sb
    for i in range(3):
        c1, s1 = nv.pack(codes[i], scales[i])
        assert np.array_equal(pc[i * cb:(i + 1) * cb], c1)
        assert np.array_equal(ps[i * sb:(i + 1) * sb], s1)


def test_quantize_rejects_bad_arguments_before_launch():
    q = nv.lib().nvfp4_quantize
    assert q(None, 4, 64, 64, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE
    assert q(0x3000, 0, 64, 64, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE
    assert q(0x3000, 4, 24, 24, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE   # K % 16
    assert q(0x3000, 4, 64, 32, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE   # ld < K
    assert q(0x3000, 4, 64, 66, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE   # ld % 4
    assert q(0x3004, 4, 64, 64, 0x1000, 0x2000, None) == nv.ERR_MISALIGNED
    assert q(0x3000, 4, 64, 64, 0x1008, 0x2000, None) == nv.ERR_MISALIGNED


def test_quantize_bf16_rejects_bad_arguments_before_launch():
    """The bfloat16 entry point: the same rules, rows of 8-element multiples."""
    q = nv.lib().nvfp4_quantize_bf16
    assert q(None, 4, 64, 64, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE
    assert q(0x3000, 0, 64, 64, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE
    assert q(0x3000, 4, 24, 24, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE   # K % 16
    assert q(0x3000, 4, 64, 32, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE   # ld < K
    assert q(0x3000, 4, 64, 68, 0x1000, 0x2000, None) == nv.ERR_INVALID_VALUE   # ld % 8
    assert q(0x3008, 4, 64, 64, 0x1000, 0x2000, None) == nv.ERR_MISALIGNED
    assert q(0x3000, 4, 64, 64, 0x1000, 0x2004, None) == nv.ERR_MISALIGNED


def test_gemm_quantized_rejects_bad_arguments_before_launch():
    """nvfp4_gemm_quantized: the GEMM's rules plus the activation rows' own
    (element type, row stride, at most 4 rows, rows x Kp within LDS)."""
    f = nv.lib().nvfp4_gemm_quantized

    def call(x=0x1000, t=nv.INPUT_F32, ld=64, b=0x3000, sb=0x4000, out=0x5000, M=1, N=8, K=64):
        return f(x, t, ld, b, sb, 1.0, out, M, N, K, None)
    assert call(x=None) == nv.ERR_INVALID_VALUE
    assert call(out=None) == nv.ERR_INVALID_VALUE
    assert call(t=2) == nv.ERR_INVALID_VALUE
    assert call(M=0) == nv.ERR_INVALID_VALUE
    assert call(K=24, ld=24) == nv.ERR_INVALID_VALUE            # K % 16
    assert call(ld=32) == nv.ERR_INVALID_VALUE                  # ld < K
    assert call(ld=66) == nv.ERR_INVALID_VALUE                  # fp32 rows: ld % 4
    assert call(t=nv.INPUT_BF16, ld=68) == nv.ERR_INVALID_VALUE  # bfloat16 rows: ld % 8
    assert call(x=0x1008) == nv.ERR_MISALIGNED
    assert call(b=0x3004) == nv.ERR_MISALIGNED
    assert call(M=5) == nv.ERR_UNSUPPORTED                      # decode rows only
    assert call(M=1, K=65664, ld=65664) == nv.ERR_UNSUPPORTED   # 1 x 65664 > 65536 in LDS
    assert call(M=3, K=16512, ld=16512) == nv.ERR_UNSUPPORTED   # rounded to 4 rows


def test_python_gemm_rejects_k_mismatch():
    a = nv.PackedOperand(None, None, 4, 128)
    b = nv.PackedOperand(None, None, 4, 256)
    with pytest.raises(ValueError, match="K dimension mismatch"):
        nv.gemm(a, b)


def test_plan(no_table):
    """The library's own rules (no tuned table loaded)."""
    def key(M, N, K):
        p = nv.plan(M, N, K)
        return nv.PATH_NAMES[p["path"]], p["tile"], p["split_k"]
    # dot products only for at most 2048 outputs of one or two rows
    assert key(1, 768, 6144)[0] == "gemv"
    assert key(1, 2048, 6144)[0] == "gemv"
    assert key(2, 768, 6144)[0] == "gemv"
    assert key(2, 2048, 6144)[0] == "skinny"
    assert key(4, 256, 6144)[0] == "skinny"
    assert key(16, 256, 6144)[0] == "skinny"
    # 256 x 256 tiles once they give 3/4 of a workgroup per CU, split in
    # two from half a workgroup per CU
    assert key(16384, 8192, 8192) == ("tile", 256, 1)
    assert key(2048, 6144, 6144) == ("tile", 256, 1)          # 192 tiles
    assert key(4096, 2048, 6144) == ("tile", 256, 2)          # 128 tiles
    assert key(1024, 8192, 8192) == ("tile", 256, 2)
    # below that the mid-size kernel, also where 128 x 128 tiles would number
    # 192-511 (each expectation the fastest plan measured for the shape)
    assert key(1024, 6144, 6144) == ("wsplit", 128, 1)
    assert key(2048, 2048, 6144) == ("wsplit", 128, 1)
    assert key(8192, 768, 6144) == ("wsplit", 128, 1)
    assert key(16384, 256, 6144) == ("wsplit", 128, 1)
    # else waves split K, on the tile and split of the cost estimate (tile
    # codes: 128 = 128 x 64, 64 = 64 x 64, 32 = 64 x 32, 16 = 32 x 32); each
    # expectation is the fastest plan measured for the shape
    assert key(1024, 2048, 6144) == ("wsplit", 128, 1)        # 256 tiles of 128 x 64
    assert key(2048, 768, 6144) == ("wsplit", 128, 1)
    assert key(512, 2048, 6144) == ("wsplit", 64, 1)          # 256 tiles of 64 x 64
    assert key(1024, 768, 6144) == ("wsplit", 64, 1)
    assert key(512, 768, 6144) == ("wsplit", 32, 1)           # 192 tiles of 64 x 32
    assert key(256, 2048, 6144) == ("wsplit", 32, 1)
    assert key(64, 6144, 6144) == ("wsplit", 32, 1)
    assert key(256, 768, 6144) == ("wsplit", 16, 1)           # 192 tiles of 32 x 32
    assert key(512, 256, 6144) == ("wsplit", 16, 1)
    assert key(128, 256, 6144) == ("wsplit", 16, 1)           # 32 tiles, still unsplit
    assert key(200, 300, 2048) == ("wsplit", 16, 1)
    # K split only for long K on few tiles (64 x 256 x 16384: 16 tiles)
    assert key(64, 256, 16384)[:2] == ("wsplit", 16) and 4 <= key(64, 256, 16384)[2] <= 8
    # skinny up to 16 rows while N <= 4096 and 32 rows while N <= 1024, with
    # 2-4 row blocks and up to 64 column groups K splits 3 or 4 ways
    assert key(16, 256, 6144) == ("skinny", 0, 1)
    assert key(16, 2048, 6144)[0] == "skinny"
    assert key(32, 256, 6144) == ("skinny", 0, 3)
    assert key(32, 768, 6144)[0] == "skinny"
    # past those, 32 x 32 tiles of the mid-size kernel
    for M, N in [(1, 6144), (16, 6144), (32, 2048), (48, 768), (64, 768), (64, 2048)]:
        assert key(M, N, 6144) == ("wsplit", 16, 1), (M, N)
    for M, N, K in [(512, 768, 6144), (512, 2048, 6144), (300, 5000, 64), (128, 64, 4096),
                    (64, 256, 16384), (40, 100, 65536)]:
        p = nv.plan(M, N, K)
        assert p["path"] == nv.PATH_WSPLIT and 1 <= p["split_k"] <= 8
        # split K only while every workgroup keeps a CU to itself
        tiles = -(-M // p["tile_m"]) * -(-N // p["tile_n"])
        assert p["split_k"] == 1 or tiles * p["split_k"] <= 256
    assert all(nv.plan(M, N, K)["source"] == nv.PLAN_HEURISTIC
               for M, N, K in [(1, 768, 6144), (4096, 2048, 6144), (16384, 8192, 8192)])


def test_sequence_state_and_validation():
    """Host-side rules of recorded sequences (no device needed): argument
    checks at add time, nothing to finalize when empty, no launch before
    finalize, NULL handles."""
    lib = nv.lib()
    h = nv._vp()
    assert lib.nvfp4_sequence_create(None) == nv.ERR_INVALID_VALUE
    assert lib.nvfp4_sequence_create(ctypes.byref(h)) == nv.OK and h.value
    try:
        add = lib.nvfp4_sequence_add_gemm
        assert add(h, 0x1000, 0x2000, 0x3000, 0x4000, 1.0, 0x5000, 4, 4, 24) == nv.ERR_INVALID_VALUE
        assert add(h, 0x1004, 0x2000, 0x3000, 0x4000, 1.0, 0x5000, 4, 4, 64) == nv.ERR_MISALIGNED
        assert add(h, None, 0x2000, 0x3000, 0x4000, 1.0, 0x5000, 4, 4, 64) == nv.ERR_INVALID_VALUE
        g = lib.nvfp4_sequence_add_grouped_gemm
        assert g(h, 0x1000, 0x2000, 0x3000, 0x4000, 0x6002, 2, 1.0, 0x5000, 4, 4, 64) \
            == nv.ERR_MISALIGNED
        q = lib.nvfp4_sequence_add_quantize
        assert q(h, 0x3000, 4, 64, 32, 0x1000, 0x2000) == nv.ERR_INVALID_VALUE
        qb = lib.nvfp4_sequence_add_quantize_bf16
        assert qb(h, 0x3000, 4, 64, 68, 0x1000, 0x2000) == nv.ERR_INVALID_VALUE   # ld % 8
        gq = lib.nvfp4_sequence_add_gemm_quantized
        assert gq(h, 0x3000, nv.INPUT_F32, 64, 0x1000, 0x2000, 1.0, 0x5000, 5, 8, 64) \
            == nv.ERR_UNSUPPORTED
        # nothing recorded: nothing to finalize; not finalized: no launch
        assert lib.nvfp4_sequence_finalize(h) == nv.ERR_INVALID_VALUE
        assert lib.nvfp4_sequence_launch(h, None) == nv.ERR_STATE
        assert add(h, 0x1000, 0x2000, 0x3000, 0x4000, 1.0, 0x5000, 4, 4, 64) == nv.OK
        assert q(h, 0x3000, 4, 64, 64, 0x1000, 0x2000) == nv.OK
        assert qb(h, 0x3000, 4, 64, 72, 0x1000, 0x2000) == nv.OK
        assert gq(h, 0x3000, nv.INPUT_BF16, 72, 0x1000, 0x2000, 1.0, 0x5000, 2, 8, 64) == nv.OK
        assert g(h, 0x1000, 0x2000, 0x3000, 0x4000, 0x6000, 2, 1.0, 0x5000, 0, 4, 64) == nv.OK
    finally:
        assert lib.nvfp4_sequence_destroy(h) == nv.OK
    for f in ("nvfp4_sequence_finalize", "nvfp4_sequence_launch"):
        args = (None,) if f.endswith("finalize") else (None, None)
        assert getattr(lib, f)(*args) == nv.ERR_INVALID_VALUE
    assert lib.nvfp4_sequence_destroy(None) == nv.OK
    assert lib.nvfp4_sequence_add_gemm(None, 0x1000, 0x2000, 0x3000, 0x4000, 1.0, 0x5000, 4, 4,
                                       64) == nv.ERR_INVALID_VALUE



def test_probe_arguments_are_checked_before_launch():
    """The measurement aids refuse out-of-range arguments on the host (no
    launch happens, so this runs without a GPU)."""
    L = nv.lib()
    assert L.nvfp4_probe_empty(0, 64, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_empty(1, 0, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_empty(1, 1025, None) == nv.ERR_INVALID_VALUE
    buf = ctypes.create_string_buffer(64)
    p = ctypes.addressof(buf)
    assert L.nvfp4_probe_chase(None, 16, 1, p, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_chase(p, 16, 1, None, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_chase(p, 12, 1, p, None) == nv.ERR_INVALID_VALUE   # not a power of two
    assert L.nvfp4_probe_chase(p, 0, 1, p, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_chase(p, 16, -1, p, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_chase(p, (1 << 32) + 2, 1, p, None) == nv.ERR_INVALID_VALUE
    out = ctypes.create_string_buffer(64 * 1024)
    q = ctypes.addressof(out)
    assert L.nvfp4_probe_mfma(0, 1, q, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_mfma(1, 0, q, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_mfma(1, 1, None, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_read(p, 64, 1, None, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_read(None, 64, 1, p, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_read(p, 40, 1, p, None) == nv.ERR_INVALID_VALUE    # not whole 16-byte chunks
    assert L.nvfp4_probe_read(p, 64, 0, p, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_probe_read(p + 4, 64, 1, p, None) == nv.ERR_INVALID_VALUE  # misaligned


def test_device_flags_and_poll_hook_on_the_host():
    L = nv.lib()
    assert L.nvfp4_device_flags(None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_debug_set_handoff_polls(0) == nv.OK
    assert L.nvfp4_debug_set_handoff_polls(0xFFFFFFFF) == nv.OK
    assert "flag" in nv.status_string(nv.ERR_DEVICE_FLAGS)


def test_plan_rules_on_random_shapes(no_table):
    """The library's own rules (no tuned table) on 3000 seeded random shapes:
    every plan names a tile its path has, splits K only while every slice
    keeps a CU of its own (skinny: at most 16 ways) with at least one
    64-element panel per wave, and the skinny and gemv paths only take the
    rows they can."""
    rng = np.random.Generator(np.random.PCG64(2024))
    wsplit_tiles = {(32, 32), (64, 32), (64, 64), (128, 64)}
    for _ in range(3000):
        M = int(rng.choice([rng.integers(1, 65), rng.integers(1, 4097), rng.integers(1, 20000)]))
        N = int(rng.choice([rng.integers(1, 300), rng.integers(1, 9000)]))
        K = 16 * int(rng.choice([rng.integers(1, 40), rng.integers(1, 1100)]))
        p = nv.plan(M, N, K)
        path, tm, tn, s = p["path"], p["tile_m"], p["tile_n"], p["split_k"]
        panels = -(-K // 64)
        assert 1 <= s <= max(1, -(-K // 128)), (M, N, K, p)
        if path == nv.PATH_GEMV:
            assert M <= 2 and M * N <= 2048 and s == 1, (M, N, K, p)
        elif path == nv.PATH_SKINNY:
            assert M <= 32 and s <= 16, (M, N, K, p)
        elif path == nv.PATH_WSPLIT:
            assert (tm, tn) in wsplit_tiles and p["tile"] == tm * tn // 64, (M, N, K, p)
            tiles = -(-M // tm) * -(-N // tn)
            assert s <= 8 and (s == 1 or (tiles * s <= 256 and 8 * s <= panels)), (M, N, K, p)
        else:
            assert path == nv.PATH_TILE and tm == tn == p["tile"] == 256, (M, N, K, p)
            assert s in (1, 2), (M, N, K, p)
