"""GPU test of the allocation-free entry point, nvfp4_gemm_noalloc, through
the C ABI: its output equals nvfp4_gemm's (same plan, same kernels) and the
oracle's, on two calls in a row whose second is smaller, for shapes whose
plans split K (so the static scratch is used) and one that does not; a shape
that needs more scratch than the static array holds is refused before
anything is enqueued.  Run alone in a fresh process and after the other GPU
tests."""
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


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def bits_of(t):
    return t.view(torch.int16).cpu().numpy().astype(np.uint16)


# (first, second): the second call is smaller; every plan splits K (long K
# on few 32 x 32 tiles of the mid-size kernel, or the skinny kernel)
PAIRS = [((64, 200, 16384), (48, 200, 16384)),
         ((32, 200, 6144), (20, 100, 6144)),
         ((40, 100, 65536), (24, 100, 32768))]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemm_twice(first, second):
    o = orc.load()
    for i, (M, N, K) in enumerate((first, second)):
        need, fits = nv.noalloc_scratch_bytes(M, N, K)
        p = nv.plan(M, N, K)
        say(f"call {i}: {M}x{N}x{K} plan {nv.PATH_NAMES[p['path']]} split {p['split_k']} "
            f"scratch {need} B")
        assert fits and p["split_k"] > 1 and need > 0
        ops = synth.quantized_operands(4000 + 7 * M + N, M, N, K, alpha=0.75)
        a = nv.to_device(ops.a_codes, ops.a_scales)
        b = nv.to_device(ops.b_codes, ops.b_scales)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ref = nv.gemm(a, b, ops.alpha)
        nv.gemm_noalloc(a, b, ops.alpha, out=out)
        torch.cuda.synchronize()
        g, r = bits_of(out), bits_of(ref)
        bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
        vs_gemm = compare(g, r, exact, mag, ops.alpha)
        vs_oracle = compare(g, bits, exact, mag, ops.alpha)
        say(f"  vs nvfp4_gemm {vs_gemm}; vs oracle {vs_oracle}")
        assert vs_gemm["over"] == 0 and vs_gemm["bit_exact_frac"] == 1.0, vs_gemm
        assert vs_oracle["over"] == 0 and not vs_oracle["all_zero"], vs_oracle
    assert nv.device_flags() == 0


def test_noalloc_without_split_and_refusal():
    o = orc.load()
    ops = synth.quantized_operands(4100, 1, 768, 2048, alpha=0.5)
    a, b = nv.to_device(ops.a_codes, ops.a_scales), nv.to_device(ops.b_codes, ops.b_scales)
    assert nv.noalloc_scratch_bytes(1, 768, 2048) == (0, True)
    out = nv.gemm_noalloc(a, b, ops.alpha)
    torch.cuda.synchronize()
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(bits_of(out), bits, exact, mag, ops.alpha)
    say(f"1x768x2048 without split: {r}")
    assert r["over"] == 0 and not r["all_zero"]
    # a tail round of 6144^3 needs 64 MiB of partial tiles: more than the array
    # holds (the refusal itself, before any device call, is a CPU test)
    need, fits = nv.noalloc_scratch_bytes(6144, 6144, 6144)
    say(f"6144^3 needs {need} B of scratch: fits={fits}")
    assert not fits and need > nv.NOALLOC_SCRATCH_BYTES
