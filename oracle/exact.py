"""Exact rational brute force for tiny NVFP4 GEMMs (Python ``fractions``).

TEST INFRASTRUCTURE ONLY.  This is a second, independent statement of the
same definition as the C oracle, written with exact rationals so that no
floating-point step can hide a mistake: every element decode, product, sum,
the alpha multiply and the single rounding to bfloat16 are exact.  Use it for
shapes of a few elements only (pure-Python loops).

Definition (per output element):
    C[m][n] = bf16_rne(alpha * sum_k e2m1(A[m][k]) * e4m3(SA[m][k/16])
                                    * e2m1(B[n][k]) * e4m3(SB[n][k/16]))
Two FP4 codes per byte and one FP8 scale per 16 elements: "Peeling the Kernel
Onion", section "The Benchmark Design"; alpha and the output tensor: same
page, section "The Chain of Reasoning".  Element formats: OCP Microscaling
Formats (MX) v1.0 (FP4 E2M1, FP8 E4M3 "FN").
"""
from __future__ import annotations

from fractions import Fraction


def e2m1_exact(code: int) -> Fraction:
    """FP4 E2M1: sign bit 3; exponent bits 2:1 with bias 1; mantissa bit 0."""
    sign = -1 if code & 0x8 else 1
    exp_field = (code >> 1) & 0x3
    man = code & 0x1
    if exp_field == 0:
        mag = Fraction(man, 2)                      # subnormal: 0.m x 2^(1-1)
    else:
        mag = Fraction(2 + man, 2) * Fraction(2) ** (exp_field - 1)
    return sign * mag


def e4m3_exact(byte: int):
    """FP8 E4M3 (FN variant): sign bit 7; exponent bits 6:3 with bias 7;
    mantissa bits 2:0; exponent 0 is subnormal; 0x7F / 0xFF are NaN (None)."""
    sign = -1 if byte & 0x80 else 1
    exp_field = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp_field == 0xF and man == 0x7:
        return None
    if exp_field == 0:
        mag = Fraction(man, 8) * Fraction(2) ** (1 - 7)
    else:
        mag = Fraction(8 + man, 8) * Fraction(2) ** (exp_field - 7)
    return sign * mag


def _floor_log2(x: Fraction) -> int:
    """Largest e with 2^e <= x, for x > 0 (exact)."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def bf16_round_exact(x: Fraction, negative_zero: bool = False) -> int:
    """Round an exact rational once to bfloat16, nearest with ties to even;
    returns the 16-bit pattern.  Magnitudes that round to 2^128 or above
    become infinity."""
    if x == 0:
        return 0x8000 if negative_zero else 0x0000
    sign = 0x8000 if x < 0 else 0
    ax = abs(x)
    e = max(_floor_log2(ax), -126)
    quantum = Fraction(2) ** (e - 7)
    q = round(ax / quantum)            # Fraction.__round__ rounds half to even
    v = q * quantum
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    if v < Fraction(2) ** -126:
        return sign | int(v / Fraction(2) ** -133)
    ev = _floor_log2(v)
    mant = int((v / Fraction(2) ** ev - 1) * 128)
    return sign | ((ev + 127) << 7) | mant


def _element(codes, scales, r: int, k: int):
    byte = codes[r][k // 2]
    code = (byte >> 4) if (k % 2) else (byte & 0xF)
    return e2m1_exact(code), e4m3_exact(scales[r][k // 16])


def gemm_exact(a_codes, a_scales, b_codes, b_scales, alpha, M: int, N: int, K: int):
    """Canonical operands as nested lists or arrays of ints; alpha as a float
    or Fraction.  Returns (bits[M][N], exact[M][N] as Fraction, or None where
    a NaN scale is involved; T[M][N] as Fraction)."""
    alpha = Fraction(alpha)
    bits = [[0] * N for _ in range(M)]
    exact = [[None] * N for _ in range(M)]
    mags = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            total = Fraction(0)
            mag = Fraction(0)
            nan = False
            for k in range(K):
                ca, sa = _element(a_codes, a_scales, m, k)
                cb, sb = _element(b_codes, b_scales, n, k)
                if sa is None or sb is None:
                    nan = True
                    continue
                p = ca * sa * cb * sb
                total += p
                mag += abs(p)
            if nan:
                bits[m][n] = 0x7FC0
                continue
            y = alpha * total
            exact[m][n] = y
            mags[m][n] = mag
            # An exactly-zero result is reported as +0; callers compare zero
            # results by value, not by sign bit.
            bits[m][n] = bf16_round_exact(y)
    return bits, exact, mags


def grouped_gemm_exact(a_codes, a_scales, b_codes, b_scales, offsets, alpha, N: int, K: int):
    """Grouped GEMM brute force: output row r belongs to the group g with
    offsets[g] <= r < offsets[g+1] (found by scanning the table), and its
    elements are the exact dot products with that group's weight rows
    b_codes[g], b_scales[g].  Returns bits[M][N] (same conventions as
    gemm_exact)."""
    M = int(offsets[-1])
    bits = [[0] * N for _ in range(M)]
    for r in range(M):
        g = 0
        while not (offsets[g] <= r < offsets[g + 1]):
            g += 1
        rb, _, _ = gemm_exact([a_codes[r]], [a_scales[r]], b_codes[g], b_scales[g], alpha, 1, N, K)
        bits[r] = rb[0]
    return bits
