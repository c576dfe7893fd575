"""Recorded sequences (nvfp4_sequence_*): a decode step's calls replayed with
one graph launch give, on every replay, the results of the same eager calls
bit for bit, with the program's own eager work and new inputs between the
replays; plus the state rules that need a device, and the capture guard of
the eager entry points."""
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


def bits(t):
    return t.view(torch.int16).cpu().numpy().astype(np.uint16)


class Step:
    """One decode step: quantise the fp32 activations of 16 tokens and of 1
    token, an MoE up-projection share (16 x 256 x 6144, skinny), an
    attention projection (1 x 768 x 6144, dot products), a 48 x 200 x 16384
    GEMM whose plan splits K across workgroups (long K on few tiles: the
    workspace is used), a grouped GEMM of the 16
    tokens routed to 2 of 8 experts (the decode kernel), and one of 256
    tokens routed to 2 of 8 experts (about 64 rows per expert: the mid-size
    kernel)."""

    def __init__(self, seed):
        g = torch.Generator(device=DEV).manual_seed(seed)
        K, KM = 6144, 16384
        self.x16 = torch.randn((16, K), generator=g, device=DEV)
        self.x1 = torch.randn((1, K), generator=g, device=DEV)
        self.x48 = torch.randn((48, KM), generator=g, device=DEV)
        self.w_up = nv.quantize(torch.randn((256, K), generator=g, device=DEV))
        self.w_attn = nv.quantize(torch.randn((768, K), generator=g, device=DEV) * 0.02)
        self.w_mid = nv.quantize(torch.randn((200, KM), generator=g, device=DEV))
        gops = synth.grouped_operands(seed, 16, 8, 2, 64, K, alpha=0.75)
        self.experts = nv.groups_to_device(gops.b_codes, gops.b_scales, DEV)
        self.offsets = torch.from_numpy(gops.offsets).to(DEV)
        self.tok = gops.M                       # 32 routed rows
        self.xg = torch.randn((self.tok, K), generator=g, device=DEV)
        gops2 = synth.grouped_operands(seed + 1, 256, 8, 2, 96, K, alpha=-0.5)
        self.experts2 = nv.groups_to_device(gops2.b_codes, gops2.b_scales, DEV)
        self.offsets2 = torch.from_numpy(gops2.offsets).to(DEV)
        self.tok2 = gops2.M                     # 512 routed rows
        self.xg2 = torch.randn((self.tok2, K), generator=g, device=DEV)
        mk = lambda r, k=K: nv.PackedOperand(*(torch.empty(n, dtype=torch.uint8, device=DEV)
                                               for n in nv.packed_size(r, k)), r, k)
        self.a16, self.a1, self.a48, self.ag = mk(16), mk(1), mk(48, KM), mk(self.tok)
        self.ag2 = mk(self.tok2)
        self.out = {
            "up": torch.empty((16, 256), dtype=torch.bfloat16, device=DEV),
            "attn": torch.empty((1, 768), dtype=torch.bfloat16, device=DEV),
            "mid": torch.empty((48, 200), dtype=torch.bfloat16, device=DEV),
            "moe": torch.empty((self.tok, 64), dtype=torch.bfloat16, device=DEV),
            "moe_mid": torch.empty((self.tok2, 96), dtype=torch.bfloat16, device=DEV),
        }

    def eager(self, stream=None):
        nv.quantize(self.x16, out=self.a16, stream=stream)
        nv.quantize(self.x1, out=self.a1, stream=stream)
        nv.quantize(self.x48, out=self.a48, stream=stream)
        nv.quantize(self.xg, out=self.ag, stream=stream)
        nv.gemm(self.a16, self.w_up, 1.0, out=self.out["up"], stream=stream)
        nv.gemm(self.a1, self.w_attn, 0.5, out=self.out["attn"], stream=stream)
        nv.gemm(self.a48, self.w_mid, -1.25, out=self.out["mid"], stream=stream)
        nv.grouped_gemm(self.ag, self.experts, self.offsets, 0.75, out=self.out["moe"],
                        stream=stream)
        nv.quantize(self.xg2, out=self.ag2, stream=stream)
        nv.grouped_gemm(self.ag2, self.experts2, self.offsets2, -0.5, out=self.out["moe_mid"],
                        stream=stream)

    def record(self) -> nv.Sequence:
        s = nv.Sequence()
        s.add_quantize(self.x16, self.a16)
        s.add_quantize(self.x1, self.a1)
        s.add_quantize(self.x48, self.a48)
        s.add_quantize(self.xg, self.ag)
        s.add_gemm(self.a16, self.w_up, self.out["up"], 1.0)
        s.add_gemm(self.a1, self.w_attn, self.out["attn"], 0.5)
        s.add_gemm(self.a48, self.w_mid, self.out["mid"], -1.25)
        s.add_grouped_gemm(self.ag, self.experts, self.offsets, self.out["moe"], 0.75)
        s.add_quantize(self.xg2, self.ag2)
        s.add_grouped_gemm(self.ag2, self.experts2, self.offsets2, self.out["moe_mid"], -0.5)
        return s

    def results(self):
        torch.cuda.synchronize()
        return {k: bits(v) for k, v in self.out.items()}

    def clear(self):
        for v in self.out.values():
            v.fill_(float("nan"))


def test_sequence_replays_match_eager_calls():
    step = Step(31)
    plans = {k: nv.plan(*shape) for k, shape in
             [("up", (16, 256, 6144)), ("attn", (1, 768, 6144)), ("mid", (48, 200, 16384))]}
    say(f"sequence plans {plans}")
    assert plans["mid"]["split_k"] > 1          # the sequence's own workspace is used
    seq = step.record()
    seq.finalize()
    assert seq.calls == 10
    stream = torch.cuda.Stream()
    for replay in range(4):
        # new activations, written by the program's own eager work
        with torch.no_grad():
            for x in (step.x16, step.x1, step.x48, step.xg, step.xg2):
                x.normal_()
                x.mul_(1.0 + replay)
        torch.cuda.synchronize()
        step.clear()
        step.eager()
        want = step.results()
        step.clear()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            seq.launch(stream)
        stream.synchronize()
        got = step.results()
        for k in want:
            same = np.array_equal(got[k], want[k])
            say(f"replay {replay} {k}: identical to eager = {same}")
            assert same, k
        assert not np.all(want["up"] == 0)
    # one replay against the oracle: quantise on the host, GEMM in fp64
    o = orc.load()
    ac, as_ = o.quantize(step.x16.cpu().numpy())
    wc, ws = nv.unpack(step.w_up.codes.cpu().numpy(), step.w_up.scales.cpu().numpy(), 256, 6144)
    ob, oe, om = o.gemm(ac, as_, wc, ws, 1.0)
    r = compare(got["up"], ob, oe, om, 1.0)
    say(f"sequence vs oracle (up-projection): {r}")
    assert r["over"] == 0 and r["bit_exact_frac"] >= 0.999
    seq.close()


def test_sequence_state_on_device():
    step = Step(7)
    seq = nv.Sequence()
    seq.add_gemm(step.a16, step.w_up, step.out["up"])
    seq.finalize()
    with pytest.raises(nv.Nvfp4Error) as e:
        seq.finalize()
    assert e.value.status == nv.ERR_STATE
    with pytest.raises(nv.Nvfp4Error) as e:
        seq.add_gemm(step.a16, step.w_up, step.out["up"])
    assert e.value.status == nv.ERR_STATE
    seq.launch()
    torch.cuda.synchronize()
    seq.close()


# (the refused call enqueues nothing, so torch warns that its graph is empty)
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_eager_call_under_capture_needs_its_workspace_first():
    """Under stream capture the split-K workspace cannot be created: the call
    reports NVFP4_ERR_CAPTURE and enqueues nothing; after one eager call on
    that stream the same call captures and replays correctly."""
    step = Step(5)
    nv.quantize(step.x48, out=step.a48)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    assert nv.plan(48, 200, 16384)["split_k"] > 1
    g = torch.cuda.CUDAGraph()
    with pytest.raises(nv.Nvfp4Error) as e:
        with torch.cuda.graph(g, stream=s):
            nv.gemm(step.a48, step.w_mid, 1.0, out=step.out["mid"], stream=s)
    assert e.value.status == nv.ERR_CAPTURE
    with torch.cuda.stream(s):
        nv.gemm(step.a48, step.w_mid, 1.0, out=step.out["mid"], stream=s)
    s.synchronize()
    want = bits(step.out["mid"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        nv.gemm(step.a48, step.w_mid, 1.0, out=step.out["mid"], stream=s)
    for _ in range(3):
        step.clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(step.out["mid"]), want)


def test_sequence_with_two_launch_tile_call():
    """A call whose plan runs as two launches (256 x 256 tiles, the last
    round split along K: 384 tiles) inside a recorded sequence: replays equal
    the eager call bit for bit."""
    M, N, K = 4096, 6144, 512
    p = nv.plan(M, N, K)
    assert p["tail_tiles"] > 0, p
    g = torch.Generator(device=DEV).manual_seed(99)
    x = torch.randn((M, K), generator=g, device=DEV)
    a = nv.quantize(x)
    b = nv.quantize(torch.randn((N, K), generator=g, device=DEV))
    out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    nv.gemm(a, b, 0.5, out=out)
    torch.cuda.synchronize()
    want = bits(out)
    seq = nv.Sequence()
    seq.add_gemm(a, b, out, 0.5)
    seq.finalize()
    for replay in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        seq.launch()
        torch.cuda.synchronize()
        same = np.array_equal(bits(out), want)
        say(f"two-launch call in a sequence, replay {replay}: identical = {same}")
        assert same
    seq.close()
