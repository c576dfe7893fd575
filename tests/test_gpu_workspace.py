"""GPU tests of the split-K workspace and the hand-off error flag, through
the C ABI.

* A graph captured from a split-K call keeps the workspace buffers it was
  captured with: growing the stream's workspace for a larger shape afterwards
  retires the old buffers instead of freeing them, so replaying the graph
  still gives the oracle's result.
* A two-way split-K hand-off that runs out of polls leaves its tile
  unwritten, raises the device's hand-off flag and leaves the counters ready
  for the next call.  The give-up is forced from the host (a poll budget of
  zero), so every kernel still ends normally.
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


def say(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def o():
    return orc.load()


def bits_of(t):
    return t.view(torch.int16).cpu().numpy().astype(np.uint16)


def oracle_check(o, ops, g, label):
    bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    r = compare(g, bits, exact, mag, ops.alpha)
    say(f"{label}: {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999 and not r["all_zero"], r


def test_graph_survives_workspace_growth(o):
    small = synth.quantized_operands(301, 32, 96, 1024, alpha=0.5)
    big = synth.quantized_operands(302, 48, 400, 2048, alpha=1.0)
    sa, sb = (nv.to_device(small.a_codes, small.a_scales), nv.to_device(small.b_codes, small.b_scales))
    ba, bb = nv.to_device(big.a_codes, big.a_scales), nv.to_device(big.b_codes, big.b_scales)
    out_s = torch.empty((small.M, small.N), dtype=torch.bfloat16, device="cuda")
    out_b = torch.empty((big.M, big.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.Stream()
    say("eager split-K call on the stream (creates its workspace)")
    nv.gemm(sa, sb, small.alpha, out=out_s, path=nv.PATH_SKINNY, split_k=4, stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        nv.gemm(sa, sb, small.alpha, out=out_s, path=nv.PATH_SKINNY, split_k=4,
                stream=torch.cuda.current_stream())
    say("larger split-K call on the same stream (grows the workspace)")
    nv.gemm(ba, bb, big.alpha, out=out_b, path=nv.PATH_SKINNY, split_k=8, stream=stream)
    stream.synchronize()
    oracle_check(o, big, bits_of(out_b), "grown workspace, eager")
    for rep in range(3):
        out_s.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        oracle_check(o, small, bits_of(out_s), f"replay {rep} of the graph captured before growth")
    del g


def test_handoff_give_up_is_flagged_and_recovers(o):
    ops = synth.quantized_operands(303, 300, 260, 4096, alpha=1.0)
    a, b = nv.to_device(ops.a_codes, ops.a_scales), nv.to_device(ops.b_codes, ops.b_scales)
    assert nv.device_flags() == 0
    try:
        nv.set_handoff_polls(0)
        say("two-way split, 128 x 128 tiles, poll budget 0")
        out = torch.full((ops.M, ops.N), 7.0, dtype=torch.bfloat16, device="cuda")
        nv.gemm(a, b, ops.alpha, out=out, path=nv.PATH_TILE, tile=128, split_k=2)
        flags = nv.device_flags()
        say(f"flags after the forced give-up: {flags}")
        assert flags & nv.FLAG_HANDOFF
    finally:
        nv.set_handoff_polls(None)
    assert nv.device_flags() == 0   # read and cleared
    for rep in range(2):
        out = nv.gemm(a, b, ops.alpha, path=nv.PATH_TILE, tile=128, split_k=2)
        torch.cuda.synchronize()
        oracle_check(o, ops, bits_of(out), f"two-way split after the give-up, call {rep}")
        assert nv.device_flags() == 0
