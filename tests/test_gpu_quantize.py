"""GPU NVFP4 quantisation (nvfp4_quantize) against the oracle's quantiser.

Codes and scales are integers, so the bar is bit-exact: the whole packed
buffer the kernel writes (padding rows and panels included) must equal the
host packing of the oracle's canonical codes and scales.
"""
from __future__ import annotations

import os
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
import quant_pins as qp  # noqa: E402

DEV = "cuda"
HERE = os.path.dirname(os.path.abspath(__file__))


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def o():
    return orc.load()


def check_quantize(o, x: np.ndarray, label: str, ld: int | None = None):
    """Quantise x (rows x K fp32) on the GPU, with row stride ld if given,
    and compare the packed bytes with the packed oracle result."""
    rows, K = x.shape
    say(f"{label}: rows={rows} K={K} ld={ld or K}")
    if ld is None:
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    else:
        wide = np.full((rows, ld), np.nan, np.float32)   # the gap must not be read
        wide[:, :K] = x
        xd = torch.from_numpy(wide).to(DEV)[:, :K]
    q = nv.quantize(xd)
    torch.cuda.synchronize()
    gc, gs = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    oc, os_ = o.quantize(x)
    pc, ps = nv.pack(oc, os_)
    bad_c = int(np.count_nonzero(gc != pc))
    bad_s = int(np.count_nonzero(gs != ps))
    say(f"{label}: {bad_c} code bytes and {bad_s} scale bytes differ "
        f"of {pc.size} and {ps.size}")
    assert bad_c == 0 and bad_s == 0
    return q, oc, os_


@pytest.mark.parametrize("rows,K,sigma", [(130, 6160, 1.0), (64, 2048, 0.02), (1, 16, 1.0),
                                          (17, 80, 1e3), (33, 6144, 1e-3)])
def test_quantize_distributions(o, rows, K, sigma):
    g = np.random.Generator(np.random.PCG64(rows * 100 + K))
    x = (g.standard_normal((rows, K)) * sigma).astype(np.float32)
    check_quantize(o, x, f"N(0,{sigma})")


def test_quantize_wide_magnitudes(o):
    g = np.random.Generator(np.random.PCG64(7))
    x = (g.uniform(-1, 1, (48, 1024)) * 10.0 ** g.integers(-8, 8, (48, 1024))).astype(np.float32)
    check_quantize(o, x, "magnitudes 1e-8..1e8")


def test_quantize_edge_blocks(o):
    """Hand-worked blocks, every E2M1 tie at every normal scale, exact round
    trips, saturation, infinity, zero and negative-zero blocks, tiny blocks
    whose scale rounds to 0, and the scale tie at 2^-10."""
    blocks = []
    for line in open(os.path.join(HERE, "golden", "quant_hand_blocks.txt")):
        if line.startswith("#") or not line.strip():
            continue
        blocks.append([float(v) for v in line.split()[1].split(",")])
    for sb in range(0x08, 0x7F):
        s = qp.e4m3_val(sb)
        blocks.append([6.0 * s] + [t * s for t, _ in qp.TIES] + [-t * s for t, _ in qp.TIES] + [0.0])
        blocks.append([v * s for v in qp.E2M1] + [-v * s for v in qp.E2M1])
    special = np.zeros((5, 16), np.float32)
    special[0, :2] = [6.0 * 448.0 * 1.2, -6.0 * 448.0 * 3.0]
    special[1, 0] = np.inf
    special[2, 5] = -0.0
    special[3, :2] = [6.0 * 2.0 ** -10, -1e-4]
    special[4, :2] = [0.005, -0.004]
    x = np.concatenate([np.array(blocks, np.float32), special])
    pad = (-x.shape[0]) % 4
    x = np.concatenate([x, np.zeros((pad, 16), np.float32)]).reshape(-1, 64)  # 4 blocks per row
    check_quantize(o, x, "edge blocks")


def test_quantize_boundary_neighbours(o):
    """The kernel decides codes by comparing |x| with boundary * scale
    instead of dividing; probe that where it matters: for every positive
    scale byte s (subnormal and normal) and every E2M1 rounding boundary T,
    x = T*s and its 4 fp32 neighbours on each side (both signs), in blocks
    whose amax fixes the scale at s."""
    rows = []
    bounds = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    for sb in range(0x01, 0x7F):
        s = np.float32(qp.e4m3_val(sb))
        amax = np.float32(6.0) * s
        for T in bounds:
            p = np.float32(T) * s
            vals = [p]
            up = dn = p
            for _ in range(4):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(0))
                vals += [up, dn]
            vals = [amax] + vals + [-v for v in vals[:6]]   # 16 values, amax first
            rows.append(np.array(vals[:16], np.float32))
    x = np.stack(rows)
    pad = (-x.shape[0]) % 4
    x = np.concatenate([x, np.zeros((pad, 16), np.float32)]).reshape(-1, 64)
    _, oc, os_ = check_quantize(o, x, "boundary neighbours")
    # the probe is only meaningful where the scale really is s
    assert np.array_equal(os_.reshape(-1)[:126 * 7], np.repeat(np.arange(1, 0x7F), 7))


def test_quantize_strided_rows(o):
    g = np.random.Generator(np.random.PCG64(9))
    x = g.standard_normal((40, 496)).astype(np.float32)
    check_quantize(o, x, "strided rows", ld=512)


def test_quantize_then_gemm(o):
    """Activations quantised on the GPU feed nvfp4_gemm directly; the result
    equals the oracle GEMM of the oracle-quantised activations."""
    g = np.random.Generator(np.random.PCG64(11))
    M, N, K = 70, 200, 1664
    x = g.standard_normal((M, K)).astype(np.float32)
    b = synth.quantized_operands(12, N, N, K)          # B rows only
    a = nv.quantize(torch.from_numpy(x).to(DEV))
    bd = nv.to_device(b.b_codes, b.b_scales, DEV)
    c = nv.gemm(a, bd, 0.5)
    torch.cuda.synchronize()
    gbits = c.view(torch.int16).cpu().numpy().astype(np.uint16)
    ac, as_ = o.quantize(x)
    bits, exact, mag = o.gemm(ac, as_, b.b_codes, b.b_scales, 0.5)
    r = compare(gbits, bits, exact, mag, 0.5)
    say(f"quantise then GEMM: {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999, r


def test_quantize_saturation_shape_activations(o):
    """The 16384 x 8192 activations of the compute-saturation shape, every
    byte."""
    g = np.random.Generator(np.random.PCG64(1005))
    x = g.standard_normal((16384, 8192), dtype=np.float32)
    check_quantize(o, x, "16384 x 8192 activations")


# ---------------------------------------------------------------- bfloat16 input

def widen(bits: np.ndarray) -> np.ndarray:
    """The fp32 values that bfloat16 bit patterns equal (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_tensor(bits: np.ndarray, ld: int | None = None):
    """A device bfloat16 tensor holding `bits` (rows x K), row stride ld."""
    rows, K = bits.shape
    if ld is None:
        host = np.ascontiguousarray(bits)
    else:
        host = np.full((rows, ld), 0x7FC0, np.uint16)   # NaN in the gap: it must not be read
        host[:, :K] = bits
    t = torch.from_numpy(host.view(np.int16)).to(DEV).view(torch.bfloat16)
    return t if ld is None else t[:, :K]


def check_quantize_bf16(o, bits: np.ndarray, label: str, ld: int | None = None):
    """nvfp4_quantize_bf16 of bfloat16 rows against the oracle's quantiser
    of the same values widened to fp32, every packed byte."""
    rows, K = bits.shape
    say(f"{label} (bf16): rows={rows} K={K} ld={ld or K}")
    q = nv.quantize(bf16_tensor(bits, ld))
    torch.cuda.synchronize()
    gc, gs = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    oc, os_ = o.quantize(widen(bits))
    pc, ps = nv.pack(oc, os_)
    bad_c, bad_s = int(np.count_nonzero(gc != pc)), int(np.count_nonzero(gs != ps))
    say(f"{label} (bf16): {bad_c} code bytes and {bad_s} scale bytes differ")
    assert bad_c == 0 and bad_s == 0
    return q, oc, os_


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bits, round to nearest even (torch's conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rows,K,sigma", [(130, 6160, 1.0), (16, 6144, 1.0), (1, 16, 1e3),
                                          (33, 2048, 1e-3)])
def test_quantize_bf16_distributions(o, rows, K, sigma):
    g = np.random.Generator(np.random.PCG64(rows * 100 + K + 1))
    check_quantize_bf16(o, to_bf16_bits(g.standard_normal((rows, K)) * sigma), f"N(0,{sigma})")


def test_quantize_bf16_every_finite_pattern(o):
    """Every finite bfloat16 bit pattern once, shuffled into blocks (scales
    from the smallest subnormal block maxima to saturation at 448)."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    fin = allb[(allb & 0x7F80) != 0x7F80]
    g = np.random.Generator(np.random.PCG64(3))
    x = g.permutation(fin)
    x = np.concatenate([x, np.zeros((-x.size) % 64, np.uint16)]).reshape(-1, 64)
    check_quantize_bf16(o, x, "every finite pattern")


def test_quantize_bf16_boundary_neighbours(o):
    """Every positive scale byte s and E2M1 rounding boundary T: x = T*s
    (exact in bfloat16) and its 4 bfloat16 neighbours on each side, both
    signs, in blocks whose amax fixes the scale at s."""
    rows = []
    for sb in range(0x01, 0x7F):
        s = np.float32(qp.e4m3_val(sb))
        amax = to_bf16_bits(np.array([6.0 * s], np.float32))[0]
        for T in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
            p = to_bf16_bits(np.array([T * s], np.float32))[0]
            assert widen(np.array([p]))[0] == np.float32(T) * s   # exact
            vals = [int(p)] + [int(p) + d for i in range(1, 5) for d in (i, -i)]
            vals = [int(amax)] + vals + [v | 0x8000 for v in vals[:6]]
            rows.append(np.array(vals[:16], np.uint16))
    x = np.stack(rows)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 4, 16), np.uint16)]).reshape(-1, 64)
    _, _, os_ = check_quantize_bf16(o, x, "boundary neighbours")
    assert np.array_equal(os_.reshape(-1)[:126 * 7], np.repeat(np.arange(1, 0x7F), 7))


def test_quantize_bf16_strided_rows_and_sequence(o):
    """Rows with a stride past K, eagerly and recorded in a sequence: both
    equal the oracle, byte for byte."""
    g = np.random.Generator(np.random.PCG64(19))
    bits = to_bf16_bits(g.standard_normal((40, 496)))
    q, _, _ = check_quantize_bf16(o, bits, "strided rows", ld=504)
    out = nv.PackedOperand(torch.zeros_like(q.codes), torch.zeros_like(q.scales), 40, 496)
    seq = nv.Sequence()
    xd = bf16_tensor(bits, 504)
    seq.add_quantize(xd, out)
    seq.finalize()
    for rep in range(2):
        out.codes.zero_()
        out.scales.zero_()
        torch.cuda.synchronize()
        seq.launch()
        torch.cuda.synchronize()
        assert torch.equal(out.codes, q.codes) and torch.equal(out.scales, q.scales), rep
    say("strided rows (bf16): sequence replays equal the eager result")
