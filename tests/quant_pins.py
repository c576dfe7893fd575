"""Pins of the oracle's NVFP4 quantiser (oracle_quantize), each against
something other than the oracle itself: hand-worked blocks, the inputs'
own independent quantiser, exact round trips, every E2M1 tie at every normal
scale, saturation, zero and tiny blocks, sign symmetry and the rounding error
bound.  Each pin returns a list of failure messages (empty when it holds)."""
from __future__ import annotations

import os

import numpy as np

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
# E2M1 midpoints and the even code each one rounds to
TIES = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]


def e4m3_val(b: int) -> float:
    e, f = (b >> 3) & 15, b & 7
    v = (f / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return -v if b & 0x80 else v


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    c = np.empty((codes.shape[0], codes.shape[1] * 2), np.uint8)
    c[:, 0::2] = codes & 0xF
    c[:, 1::2] = codes >> 4
    return c


def pin_quant_hand_blocks(o) -> list[str]:
    bad = []
    for line in open(os.path.join(HERE, "golden", "quant_hand_blocks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, vals, sb, cb = line.split()
        x = np.array([[float(v) for v in vals.split(",")]], np.float32)
        codes, scales = o.quantize(x)
        if int(scales[0, 0]) != int(sb, 16):
            bad.append(f"{name}: scale 0x{int(scales[0, 0]):02x} != 0x{sb}")
        got = codes[0].tobytes().hex().upper()
        if got != cb:
            bad.append(f"{name}: codes {got} != {cb}")
    return bad


def pin_quant_vs_input_quantiser(o) -> list[str]:
    """The numpy quantiser of the input generator is a separate
    implementation (table midpoints and searchsorted) of the same recipe."""
    bad = []
    g = np.random.Generator(np.random.PCG64(41))
    cases = [g.standard_normal((96, 640)).astype(np.float32) * np.float32(s)
             for s in (1.0, 0.02, 300.0, 1e-3)]
    cases.append((g.uniform(-1, 1, (64, 512)) * 10.0 ** g.integers(-6, 6, (64, 512))).astype(np.float32))
    for i, x in enumerate(cases):
        c1, s1 = o.quantize(x)
        c2, s2 = synth.quantize_nvfp4(x)
        if not np.array_equal(s1, s2):
            bad.append(f"case {i}: {np.count_nonzero(s1 != s2)} scale bytes differ")
        if not np.array_equal(c1, c2):
            bad.append(f"case {i}: {np.count_nonzero(c1 != c2)} code bytes differ")
    return bad


def pin_quant_exact_roundtrip(o) -> list[str]:
    """Blocks whose values are E2M1 values times a normal E4M3 scale s, one
    of them 6 s: the quantiser returns exactly s and the codes."""
    bad = []
    g = np.random.Generator(np.random.PCG64(42))
    for sb in range(0x08, 0x7F):            # every normal scale byte (6 s stays finite)
        s = e4m3_val(sb)
        mags = g.integers(0, 8, size=16)
        mags[int(g.integers(0, 16))] = 7
        signs = g.integers(0, 2, size=16)
        x = np.array([[(-1.0 if sg else 1.0) * E2M1[m] * s for m, sg in zip(mags, signs)]],
                     np.float32)
        codes, scales = o.quantize(x)
        want = (mags | (signs << 3)).astype(np.uint8)
        if int(scales[0, 0]) != sb:
            bad.append(f"scale 0x{sb:02x}: got 0x{int(scales[0, 0]):02x}")
        if not np.array_equal(unpack_codes(codes)[0], want):
            bad.append(f"scale 0x{sb:02x}: codes {unpack_codes(codes)[0]} != {want}")
    return bad


def pin_quant_ties(o) -> list[str]:
    """x / s exactly at every E2M1 midpoint, for every normal scale s (with
    6 s in the block so the scale is s): ties go to the even code."""
    bad = []
    for sb in range(0x08, 0x7F):
        s = e4m3_val(sb)
        vals = [6.0 * s] + [t * s for t, _ in TIES] + [-t * s for t, _ in TIES] + [0.0]
        x = np.array([vals], np.float32)
        codes, scales = o.quantize(x)
        c = unpack_codes(codes)[0]
        if int(scales[0, 0]) != sb:
            bad.append(f"scale 0x{sb:02x}: got 0x{int(scales[0, 0]):02x}")
            continue
        for i, (t, want) in enumerate(TIES):
            if c[1 + i] != want or c[8 + i] != (want | 8):
                bad.append(f"scale 0x{sb:02x} tie {t}: codes {c[1 + i]}, {c[8 + i]}, want {want}")
    return bad


def pin_quant_saturation_zero_tiny(o) -> list[str]:
    bad = []
    # amax / 6 beyond 448 saturates the scale; |x / 448| beyond 6 saturates the code
    x = np.zeros((4, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0 * 448.0 * 1.2, -6.0 * 448.0 * 3.0
    x[1, 0] = np.inf
    x[2, 5] = -0.0                       # all-zero block with a negative zero
    x[3, 0] = 6.0 * 2.0 ** -10           # amax / 6 = 2^-10: halfway to the smallest subnormal
    x[3, 1] = -1e-4
    codes, scales = o.quantize(x)
    c = unpack_codes(codes)
    if int(scales[0, 0]) != 0x7E or c[0, 0] != 7 or c[0, 1] != 15:
        bad.append(f"saturation: scale 0x{int(scales[0, 0]):02x} codes {c[0, :2]}")
    if int(scales[1, 0]) != 0x7E or c[1, 0] != 7:
        bad.append(f"infinity: scale 0x{int(scales[1, 0]):02x} code {c[1, 0]}")
    if int(scales[2, 0]) != 0 or c[2, 5] != 8 or np.any(np.delete(c[2], 5) != 0):
        bad.append(f"zero block: scale 0x{int(scales[2, 0]):02x} codes {c[2]}")
    if int(scales[3, 0]) != 0 or c[3, 0] != 0 or c[3, 1] != 8:
        bad.append(f"tie with scale 0 (even byte 0x00): scale 0x{int(scales[3, 0]):02x} codes {c[3, :2]}")
    return bad


def pin_quant_sign_symmetry(o) -> list[str]:
    g = np.random.Generator(np.random.PCG64(43))
    x = g.standard_normal((64, 256)).astype(np.float32)
    c1, s1 = o.quantize(x)
    c2, s2 = o.quantize(-x)
    bad = []
    if not np.array_equal(s1, s2):
        bad.append("scales change with the sign")
    if not np.array_equal(c1 ^ 0x88, c2):
        bad.append(f"{np.count_nonzero((c1 ^ 0x88) != c2)} code bytes are not sign flips")
    return bad


def pin_quant_error_bound(o) -> list[str]:
    """Without saturation, the dequantised value is within half the local
    E2M1 spacing (times the scale) of x, up to the fp32 rounding of x / s."""
    g = np.random.Generator(np.random.PCG64(44))
    x = g.standard_normal((128, 512)).astype(np.float32)
    codes, scales = o.quantize(x)
    c = unpack_codes(codes).astype(np.int64)
    s = np.array([e4m3_val(int(b)) for b in range(256)])[scales.astype(np.int64)]
    s = np.repeat(s, 16, axis=1)
    mag = np.array(E2M1)[c & 7]
    deq = np.where(c & 8, -mag, mag) * s
    y = np.abs(x.astype(np.float64)) / np.where(s > 0, s, 1.0)
    half = np.where(y <= 2.0, 0.25, np.where(y <= 4.0, 0.5, 1.0))
    ok = (s > 0) & (y <= 6.0)
    err = np.abs(deq - x.astype(np.float64))
    lim = half * s * (1 + 2.0 ** -20)
    n = int(np.count_nonzero(ok & (err > lim)))
    return [f"{n} elements beyond the rounding bound"] if n else []


ALL_QUANT_PINS = [pin_quant_hand_blocks, pin_quant_vs_input_quantiser, pin_quant_exact_roundtrip,
                  pin_quant_ties, pin_quant_saturation_zero_tiny, pin_quant_sign_symmetry,
                  pin_quant_error_bound]
