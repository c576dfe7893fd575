"""Checks that pin the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an ``oracle.oracle.Oracle`` and returns a list
of failure messages (empty = pass).  The same functions run against the real
oracle and against builds with one planted mistake, so the test suite can
show that every such mistake fails at least one pin.

What each pin rests on:
  - E4M3 decode: torch's float8_e4m3fn conversion (a library routine);
  - E2M1 decode: the value table of the OCP MX specification
    (tests/golden/e2m1_values.txt);
  - bf16 rounding: torch's fp32 -> bfloat16 conversion (round to nearest
    even) and exact-rational rounding;
  - the GEMM: hand-worked single blocks (tests/golden/hand_blocks.txt),
    exact-rational brute force on tiny shapes, a float64 matmul of the decoded
    codes when every scale is 1, single-product (one-hot) cases, and
    invariants (zero scale, sign flip, transpose, K-block permutation, alpha
    powers of two, cancellation that fp32 accumulation would lose).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import exact as ex

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_e2m1() -> dict[int, float]:
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    assert len(vals) == 16
    return vals


def golden_hand_blocks():
    rows = []
    with open(os.path.join(GOLDEN, "hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, ac, sa, bc, sb, alpha, val, bits, mag = line.split()
            rows.append(dict(
                name=name,
                a_codes=np.frombuffer(bytes.fromhex(ac), np.uint8).reshape(1, 8).copy(),
                a_scales=np.array([[int(sa, 16)]], np.uint8),
                b_codes=np.frombuffer(bytes.fromhex(bc), np.uint8).reshape(1, 8).copy(),
                b_scales=np.array([[int(sb, 16)]], np.uint8),
                alpha=float(alpha), value=float(val), bits=int(bits, 16), mag=float(mag)))
    return rows


def torch_e4m3(byte: int) -> float:
    return float(torch.tensor([byte], dtype=torch.uint8).view(torch.float8_e4m3fn).float()[0])


def torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def same_bits_or_zero(a: int, b: int) -> bool:
    """Equal patterns, or both zero of either sign."""
    return a == b or ((a & 0x7FFF) == 0 and (b & 0x7FFF) == 0)


# ---------------------------------------------------------------- decoders

def pin_e4m3_vs_torch(o) -> list[str]:
    bad = []
    for b in range(256):
        want = torch_e4m3(b)
        got = o.e4m3(b)
        if math.isnan(want):
            if not math.isnan(got):
                bad.append(f"e4m3 0x{b:02x}: want NaN got {got}")
        elif got != want or math.copysign(1, got) != math.copysign(1, want):
            bad.append(f"e4m3 0x{b:02x}: want {want} got {got}")
    return bad


def pin_e2m1_vs_table(o) -> list[str]:
    bad = []
    for c, want in golden_e2m1().items():
        got = o.e2m1(c)
        if got != want or math.copysign(1, got) != math.copysign(1, want):
            bad.append(f"e2m1 {c}: want {want} got {got}")
    return bad


def pin_bf16_rounding(o) -> list[str]:
    bad = []
    g = np.random.Generator(np.random.PCG64(7))
    # fp32 inputs: normal, subnormal, ties (low 16 bits 0x8000), near overflow
    u = g.integers(0, 2 ** 32, size=4000, dtype=np.uint64).astype(np.uint32)
    ties = (g.integers(0, 2 ** 16, size=500, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000,
                        0x00000001, 0x80008001, 0x3F808000, 0x3F818000], np.uint32)
    bits32 = np.concatenate([u, ties, special])
    x32 = bits32.view(np.float32)
    x32 = x32[np.isfinite(x32)]
    want = torch_bf16_bits(x32)
    for x, w in zip(x32.tolist(), want.tolist()):
        got = o.bf16(float(x))
        if got != w:
            bad.append(f"bf16({x!r}): want 0x{w:04x} got 0x{got:04x}")
            if len(bad) > 10:
                break
    # fp64 values that fp32 cannot hold: exact-rational rounding decides
    d = g.standard_normal(2000) * np.ldexp(1.0, g.integers(-140, 128, size=2000))
    for x in d.tolist():
        w = ex.bf16_round_exact(Fraction(x))
        got = o.bf16(x)
        if got != w:
            bad.append(f"bf16({x!r}) exact: want 0x{w:04x} got 0x{got:04x}")
            if len(bad) > 20:
                break
    return bad


def pin_element_order(o) -> list[str]:
    """Interface convention: element 2j sits in bits 3:0 of byte j and
    element 2j+1 in bits 7:4; element k uses scale byte k // 16.  (The GEMM
    result is blind to the nibble order when both operands share it, so this
    is checked on single elements.)"""
    codes = np.array([[0x21, 0x43] + [0x00] * 14], np.uint8)   # K = 32
    scales = np.array([[0x38, 0x40]], np.uint8)                # 1.0, 2.0
    want = {0: 0.5, 1: 1.0, 2: 1.5, 3: 2.0, 16: 0.0}
    bad = [f"element {k}: {o.element(codes, scales, 0, k)} != {v}"
           for k, v in want.items() if o.element(codes, scales, 0, k) != v]
    codes2 = codes.copy()
    codes2[0, 8] = 0x07                                        # k = 16 -> 6.0 * 2.0
    if o.element(codes2, scales, 0, 16) != 12.0 or o.element(codes2, scales, 0, 17) != 0.0:
        bad.append("element 16/17 or its scale block is wrong")
    return bad


# ---------------------------------------------------------------- GEMM

def pin_hand_blocks(o) -> list[str]:
    bad = []
    for r in golden_hand_blocks():
        bits, exact, mag = o.gemm(r["a_codes"], r["a_scales"], r["b_codes"], r["b_scales"],
                                  r["alpha"])
        if not same_bits_or_zero(int(bits[0, 0]), r["bits"]):
            bad.append(f"{r['name']}: bits 0x{int(bits[0, 0]):04x} != 0x{r['bits']:04x}")
        if exact[0, 0] != r["value"]:
            bad.append(f"{r['name']}: value {exact[0, 0]} != {r['value']}")
        if mag[0, 0] != r["mag"]:
            bad.append(f"{r['name']}: sum|p| {mag[0, 0]} != {r['mag']}")
    return bad


def _finite_scale_bytes():
    return np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)


def pin_bruteforce(o, cases: int = 10000, seed: int = 11) -> list[str]:
    """Random 2x2xK problems (K in 16, 32, 48) over every code and every
    finite scale byte (negative and subnormal included), random alpha."""
    bad = []
    g = np.random.Generator(np.random.PCG64(seed))
    fin = _finite_scale_bytes()
    alphas = [1.0, 0.5, -2.0, 0.3, 1.7, -0.0078125, 3.0e-3]
    for i in range(cases):
        K = int(g.choice([16, 32, 48]))
        ac = g.integers(0, 256, size=(2, K // 2), dtype=np.uint8)
        bc = g.integers(0, 256, size=(2, K // 2), dtype=np.uint8)
        as_ = g.choice(fin, size=(2, K // 16)).astype(np.uint8)
        bs = g.choice(fin, size=(2, K // 16)).astype(np.uint8)
        alpha = float(np.float32(alphas[i % len(alphas)]))
        bits, exact_v, mag = o.gemm(ac, as_, bc, bs, alpha)
        wb, we, wm = ex.gemm_exact(ac.tolist(), as_.tolist(), bc.tolist(), bs.tolist(), alpha,
                                   2, 2, K)
        for m in range(2):
            for n in range(2):
                if not same_bits_or_zero(int(bits[m, n]), wb[m][n]):
                    bad.append(f"case {i} K={K} ({m},{n}): 0x{int(bits[m, n]):04x} != "
                               f"0x{wb[m][n]:04x}")
                if Fraction(float(mag[m, n])) != wm[m][n]:
                    bad.append(f"case {i} ({m},{n}): T {mag[m, n]} != {float(wm[m][n])}")
        if len(bad) > 10:
            break
    return bad


def pin_unit_scales_matmul(o) -> list[str]:
    """All scales 1.0 (byte 0x38): C = alpha * (codes_A . codes_B^T), which a
    float64 matmul of the table-decoded codes gives exactly at these sizes."""
    bad = []
    table = golden_e2m1()
    lut = np.array([table[c] for c in range(16)], np.float64)
    g = np.random.Generator(np.random.PCG64(5))
    for (M, N, K) in [(3, 5, 64), (7, 2, 128), (1, 9, 32)]:
        ac = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        bc = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        as_ = np.full((M, K // 16), 0x38, np.uint8)
        bs = np.full((N, K // 16), 0x38, np.uint8)

        def dec(codes):
            lo, hi = codes & 0xF, codes >> 4
            out = np.empty((codes.shape[0], codes.shape[1] * 2), np.float64)
            out[:, 0::2] = lut[lo]
            out[:, 1::2] = lut[hi]
            return out

        want_val = 0.5 * (dec(ac) @ dec(bc).T)
        want_bits = torch_bf16_bits(want_val.astype(np.float32))
        assert np.all(want_val.astype(np.float32).astype(np.float64) == want_val)
        bits, exact_v, _ = o.gemm(ac, as_, bc, bs, 0.5)
        if not np.array_equal(exact_v, want_val):
            bad.append(f"unit scales {M}x{N}x{K}: values differ")
        if not all(same_bits_or_zero(int(x), int(y)) for x, y in zip(bits.ravel(), want_bits.ravel())):
            bad.append(f"unit scales {M}x{N}x{K}: bits differ")
    return bad


def pin_onehot(o) -> list[str]:
    """A single non-zero code in A (row m, element k) and in B (row n, same k):
    the only non-zero output is the one product, at (m, n)."""
    bad = []
    table = golden_e2m1()
    g = np.random.Generator(np.random.PCG64(9))
    fin = [b for b in range(256) if (b & 0x7F) != 0x7F]
    M, N, K = 3, 4, 48
    for t in range(200):
        m, n, k = int(g.integers(M)), int(g.integers(N)), int(g.integers(K))
        ca, cb = int(g.integers(1, 16)), int(g.integers(1, 16))
        if ca == 8 or cb == 8:
            continue
        sa, sb = int(g.choice(fin)), int(g.choice(fin))
        ac = np.zeros((M, K // 2), np.uint8)
        bc = np.zeros((N, K // 2), np.uint8)
        ac[m, k // 2] = ca << (4 * (k % 2))
        bc[n, k // 2] = cb << (4 * (k % 2))
        as_ = np.full((M, K // 16), 0x38, np.uint8)
        bs = np.full((N, K // 16), 0x38, np.uint8)
        as_[m, k // 16] = sa
        bs[n, k // 16] = sb
        prod = table[ca] * torch_e4m3(sa) * table[cb] * torch_e4m3(sb)
        want = np.zeros((M, N), np.float64)
        want[m, n] = prod
        bits, exact_v, _ = o.gemm(ac, as_, bc, bs, 1.0)
        if not np.array_equal(exact_v, want):
            bad.append(f"one-hot m={m} n={n} k={k} ca={ca} cb={cb} sa={sa:#x} sb={sb:#x}")
        wb = torch_bf16_bits(np.array([prod], np.float32))[0]
        if not same_bits_or_zero(int(bits[m, n]), int(wb)):
            bad.append(f"one-hot bits m={m} n={n} k={k}")
        if len(bad) > 5:
            break
    return bad


def _rand_ops(seed, M, N, K):
    g = np.random.Generator(np.random.PCG64(seed))
    fin = _finite_scale_bytes()
    ac = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bc = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    as_ = g.choice(fin, size=(M, K // 16)).astype(np.uint8)
    bs = g.choice(fin, size=(N, K // 16)).astype(np.uint8)
    return ac, as_, bc, bs


def pin_invariants(o) -> list[str]:
    bad = []
    M, N, K = 5, 6, 96
    ac, as_, bc, bs = _rand_ops(21, M, N, K)
    base, bex, bmag = o.gemm(ac, as_, bc, bs, 1.0)
    # zero scale on A: every output is zero
    z, _, _ = o.gemm(ac, np.zeros_like(as_), bc, bs, 1.0)
    if np.any(z & 0x7FFF):
        bad.append("zero A scales give a non-zero output")
    # flipping every A code sign (xor 0x88) negates C exactly; T unchanged
    f, fex, fmag = o.gemm(ac ^ np.uint8(0x88), as_, bc, bs, 1.0)
    if not np.array_equal(fex, -bex):
        bad.append("sign flip of A codes does not negate the exact sum")
    if not np.array_equal(fmag, bmag):
        bad.append("sign flip of A codes changes sum|p|")
    nz = (base & 0x7FFF) != 0
    if not np.array_equal((f ^ 0x8000)[nz], base[nz]):
        bad.append("sign flip of A codes does not flip the output sign bit")
    # setting the sign bit of every A scale negates C exactly
    s, sex, _ = o.gemm(ac, as_ ^ np.uint8(0x80), bc, bs, 1.0)
    if not np.array_equal(sex, -bex):
        bad.append("negated A scales do not negate C")
    # transpose symmetry: gemm(B, A) = gemm(A, B)^T
    t, tex, _ = o.gemm(bc, bs, ac, as_, 1.0)
    if not np.array_equal(t, base.T) or not np.array_equal(tex, bex.T):
        bad.append("gemm(B,A) != gemm(A,B)^T")
    # permuting K-blocks together with their scales leaves C bit-identical
    perm = np.random.Generator(np.random.PCG64(3)).permutation(K // 16)
    def permute(codes, scales):
        c = codes.reshape(codes.shape[0], K // 16, 8)[:, perm, :].reshape(codes.shape)
        return np.ascontiguousarray(c), np.ascontiguousarray(scales[:, perm])
    pa, psa = permute(ac, as_)
    pb, psb = permute(bc, bs)
    p, pex, _ = o.gemm(pa, psa, pb, psb, 1.0)
    if not np.array_equal(p, base) or not np.array_equal(pex, bex):
        bad.append("K-block permutation changes C")
    # alpha = 2^z scales the exact value exactly
    for z in (-3, 1, 4):
        a2, a2ex, _ = o.gemm(ac, as_, bc, bs, 2.0 ** z)
        if not np.array_equal(a2ex, bex * 2.0 ** z):
            bad.append(f"alpha 2^{z} does not scale C exactly")
    # T >= |S| everywhere; alternating +-1 products: S = 0, T = K
    if np.any(bmag < np.abs(bex)):
        bad.append("sum|p| < |S|")
    alt_a = np.full((1, K // 2), 0xA2, np.uint8)   # +1, -1, +1, -1, ...
    one_b = np.full((1, K // 2), 0x22, np.uint8)
    ones = np.full((1, K // 16), 0x38, np.uint8)
    _, aex, amag = o.gemm(alt_a, ones, one_b, ones, 1.0)
    if aex[0, 0] != 0.0 or amag[0, 0] != float(K):
        bad.append(f"alternating +-1: S={aex[0, 0]} T={amag[0, 0]}, want 0 and {K}")
    return bad


def pin_cancellation(o) -> list[str]:
    """Block 0 holds the product 2^-20 at k=0 (codes 0.5, scales 2^-9); block 1
    holds +2688^2 at k=16 and -2688^2 at k=17.  The exact sum is 2^-20 (bf16
    0x3580); accumulating in fp32 from k=0 would lose it."""
    K = 32
    ac = np.zeros((1, K // 2), np.uint8)
    bc = np.zeros((1, K // 2), np.uint8)
    ac[0, 0] = 0x01                  # k=0: 0.5
    bc[0, 0] = 0x01
    ac[0, 8] = 0xF7                  # k=16: +6, k=17: -6
    bc[0, 8] = 0x77                  # k=16: +6, k=17: +6
    as_ = np.array([[0x01, 0x7E]], np.uint8)   # 2^-9, 448
    bs = np.array([[0x01, 0x7E]], np.uint8)
    bits, exv, _ = o.gemm(ac, as_, bc, bs, 1.0)
    bad = []
    if exv[0, 0] != 2.0 ** -20:
        bad.append(f"cancellation: S = {exv[0, 0]!r}, want 2^-20")
    if int(bits[0, 0]) != 0x3580:
        bad.append(f"cancellation: bits 0x{int(bits[0, 0]):04x}, want 0x3580")
    return bad


def pin_nan_scale(o) -> list[str]:
    ac, as_, bc, bs = _rand_ops(31, 2, 3, 32)
    ac[:] = 0x22
    bc[:] = 0x22
    as_ = as_.copy()
    as_[1, 1] = 0x7F
    bits, _, _ = o.gemm(ac, as_, bc, bs, 1.0)
    bad = []
    if not all(((int(b) & 0x7F80) == 0x7F80 and (int(b) & 0x7F) != 0) for b in bits[1]):
        bad.append("a NaN scale in row 1 of A does not give NaN in row 1 of C")
    if any(((int(b) & 0x7F80) == 0x7F80) for b in bits[0]):
        bad.append("a NaN scale in row 1 of A leaks into row 0 of C")
    return bad


def pin_points_match_full(o) -> list[str]:
    ac, as_, bc, bs = _rand_ops(41, 9, 7, 80)
    bits, exv, mag = o.gemm(ac, as_, bc, bs, 0.75)
    ms = np.repeat(np.arange(9), 7)
    ns = np.tile(np.arange(7), 9)
    pb, pe, pm = o.gemm_points(ac, as_, bc, bs, 0.75, ms, ns)
    if not (np.array_equal(pb, bits.ravel()) and np.array_equal(pe, exv.ravel())
            and np.array_equal(pm, mag.ravel())):
        return ["gemm_points differs from gemm"]
    return []




def pin_grouped_bruteforce(o, cases: int = 300, seed: int = 17, grouped=None) -> list[str]:
    """Grouped GEMM vs the exact brute force on tiny problems: 1-4 groups of
    0-3 rows each (empty groups included), N in 1..3, K in 16, 32, random
    codes and finite scales, random alpha.  ``grouped`` replaces the
    oracle's grouped_gemm (to check that this pin catches a wrong one)."""
    bad = []
    grouped = grouped or o.grouped_gemm
    g = np.random.Generator(np.random.PCG64(seed))
    fin = _finite_scale_bytes()
    for i in range(cases):
        G = int(g.integers(1, 5))
        N = int(g.integers(1, 4))
        K = int(g.choice([16, 32]))
        sizes = g.integers(0, 4, size=G)
        if sizes.sum() == 0:
            sizes[int(g.integers(0, G))] = 1
        offsets = np.zeros(G + 1, np.int64)
        offsets[1:] = np.cumsum(sizes)
        M = int(offsets[-1])
        ac = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        as_ = g.choice(fin, size=(M, K // 16)).astype(np.uint8)
        bc = g.integers(0, 256, size=(G, N, K // 2), dtype=np.uint8)
        bs = g.choice(fin, size=(G, N, K // 16)).astype(np.uint8)
        alpha = float(np.float32(g.choice([1.0, 0.5, -1.5, 0.3])))
        bits, _, _ = grouped(ac, as_, bc, bs, offsets, alpha)
        want = ex.grouped_gemm_exact(ac.tolist(), as_.tolist(), bc.tolist(), bs.tolist(),
                                     offsets.tolist(), alpha, N, K)
        for r in range(M):
            for n in range(N):
                if not same_bits_or_zero(int(bits[r, n]), want[r][n]):
                    bad.append(f"case {i} G={G} sizes={sizes.tolist()} ({r},{n}): "
                               f"0x{int(bits[r, n]):04x} != 0x{want[r][n]:04x}")
        if len(bad) > 10:
            break
    return bad


ALL_PINS = [pin_e4m3_vs_torch, pin_e2m1_vs_table, pin_element_order, pin_bf16_rounding, pin_hand_blocks,
            pin_bruteforce, pin_unit_scales_matmul, pin_onehot, pin_invariants,
            pin_cancellation, pin_nan_scale, pin_points_match_full, pin_grouped_bruteforce]


def run_all(o, quick: bool = False) -> dict[str, list[str]]:
    out = {}
    for p in ALL_PINS:
        if quick and p is pin_bruteforce:
            out[p.__name__] = p(o, cases=600)
        elif quick and p is pin_grouped_bruteforce:
            out[p.__name__] = p(o, cases=40)
        else:
            out[p.__name__] = p(o)
    return out
