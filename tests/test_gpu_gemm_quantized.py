"""GPU tests of nvfp4_gemm_quantized: the decode-sized GEMM that quantises
its fp32 or bfloat16 activation rows itself.

Two bars: bit-identity with the two-call form (nvfp4_quantize or
nvfp4_quantize_bf16, then nvfp4_gemm on the dot-product path), and parity
with the oracle (the oracle's quantiser on the rows -- widened to fp32 for
bfloat16 -- then the oracle GEMM), element by element.
"""
from __future__ import annotations

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


def bits(t) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().astype(np.uint16)


def activations(seed: int, M: int, K: int, bf16: bool, ld: int | None = None, sigma=1.0):
    """Device rows (fp32 or bfloat16, row stride ld with NaN in the gap) and
    the fp32 values they hold."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = (g.standard_normal((M, K)) * sigma).astype(np.float32)
    t = torch.from_numpy(x)
    if bf16:
        t = t.to(torch.bfloat16)
        x = t.to(torch.float32).numpy()          # the values the bfloat16 rows hold (exact)
    if ld is not None:
        wide = torch.full((M, ld), float("nan"), dtype=t.dtype)
        wide[:, :K] = t
        return wide.to(DEV)[:, :K], x
    return t.to(DEV), x


def check(o, M, N, K, bf16, seed=1, ld=None, alpha=0.5, sigma=1.0):
    label = f"{M}x{N}x{K} {'bf16' if bf16 else 'fp32'} ld={ld or K}"
    say(label)
    xd, x = activations(seed * 1000 + M * 7 + K, M, K, bf16, ld, sigma)
    w = synth.quantized_operands(seed + N + K, N, N, K, sigma_b=0.02)
    b = nv.to_device(w.b_codes, w.b_scales, DEV)
    fused = nv.gemm_quantized(xd, b, alpha)
    two = nv.gemm(nv.quantize(xd), b, alpha, path=nv.PATH_GEMV)
    torch.cuda.synchronize()
    gf, gt = bits(fused), bits(two)
    assert np.array_equal(gf, gt), f"{label}: {int(np.count_nonzero(gf != gt))} elements differ"
    ac, as_ = o.quantize(x)
    ob, oe, om = o.gemm(ac, as_, w.b_codes, w.b_scales, alpha)
    r = compare(gf, ob, oe, om, alpha)
    say(f"{label}: identical to quantize + gemm; oracle {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999 and not r["all_zero"], r


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_decode_projection(o, M, bf16):
    """The decode attention projection's shape (N = 768, K = 6144) at 1-4 rows."""
    check(o, M, 768, 6144, bf16)


@pytest.mark.parametrize("M,N,K", [(1, 16, 16), (2, 40, 80), (1, 72, 256), (3, 300, 8320),
                                   (4, 16, 16384), (1, 256, 65536)])
def test_shapes(o, M, N, K):
    """A single block, ragged N, K not a multiple of 128, two batches of
    half-panels (K > 8192), and both LDS limits (4 x 16384 and 1 x 65536)."""
    for bf16 in (False, True):
        check(o, M, N, K, bf16, seed=2)


def test_strided_rows_wide_values_and_sequence(o):
    """Row strides past K (the gap holds NaN: it must not be read), large
    values (saturated scales) and small ones (subnormal E4M3 scales; below
    amax 6 * 2^-10 a block's scale, and so the block, is zero), and a
    recorded sequence's replays."""
    check(o, 2, 136, 1024, False, ld=1040, sigma=1e3)
    check(o, 3, 136, 1024, True, ld=1032, sigma=0.05)
    xd, _ = activations(5, 2, 6144, True)
    w = synth.quantized_operands(6, 768, 768, 6144)
    b = nv.to_device(w.b_codes, w.b_scales, DEV)
    want = nv.gemm_quantized(xd, b, 0.25)
    out = torch.zeros((2, 768), dtype=torch.bfloat16, device=DEV)
    seq = nv.Sequence()
    seq.add_gemm_quantized(xd, b, 0.25, out)
    seq.finalize()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        seq.launch()
        torch.cuda.synchronize()
        assert torch.equal(out, want), rep
    say("sequence replays equal the eager call")
