#!/usr/bin/env python3
"""Benchmark of the gfx950 NVFP4 block-scaled GEMM, C = alpha * (A . B^T).

One "step" is one call of the whole path, nvfp4_gemm, on packed operands
already resident in HBM (decode, MFMA contraction, split-K reduction where the
plan uses it, alpha and bf16 epilogue).  Timing follows the protocol of
"Peeling the Kernel Onion", section "The Benchmark Design" (warm-up calls,
then timed calls bracketed by device synchronisation), with HIP events
recorded on the stream the kernels are launched on.

The headline line is the decode attention projection, M=1, N=768, K=6144,
alpha=0.5 (the pages' batch-1 point, 0.30 TFLOPS on their GPU); the other
workloads are reported under "per_shape".  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HEADLINE = 2            # decode attention projection 1 x 768 x 6144
PAGES_TFLOPS = {2: 0.30, 3: 161.0, 4: 437.0}  # same shapes, measured on the pages' GPU
# MI355X published peaks
HBM_GBPS = 8000.0
MFMA_F16_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=HEADLINE, help="1..5")
    ap.add_argument("--only-headline", action="store_true",
                    help="skip the per-shape lines for the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--grouped-only", action="store_true",
                    help="time only one grouped (all experts in one launch) workload")
    ap.add_argument("--grouped-workload", default=synth.GROUPED_CONFIGS[0].name,
                    choices=[c.name for c in synth.GROUPED_CONFIGS],
                    help="the grouped workload of --grouped-only (and of its --traffic-summary)")
    ap.add_argument("--quantize-only", action="store_true",
                    help="time only the fp32 -> NVFP4 quantisation shapes")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode step: eager calls against one recorded sequence")
    ap.add_argument("--floors-only", action="store_true",
                    help="measure only the floors (empty kernel, load latencies, measured peaks)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle baseline")
    ap.add_argument("--cold", action="store_true",
                    help="also time with operand copies rotated beyond the last-level cache")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR",
                                                           "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs of --workload into "
                         "profiles/traffic_<workload>.json (no GPU needed)")
    return ap.parse_args()


COPY_BYTES = 256 << 20   # size of the copy used to scale the HBM counters
CSRC = os.path.join(ROOT, "block_scaled_fp4_04_amd", "csrc")
# the sources whose code the counters of a workload depend on
KERNEL_SOURCES = {
    "gemm": ["nvfp4_internal.h", "nvfp4_device.h", "nvfp4_quant_device.h", "nvfp4_kernels.hip"],
    "grouped": ["nvfp4_internal.h", "nvfp4_device.h", "nvfp4_grouped.hip"],
}


def _sources_for(cfg) -> list[str]:
    kind = "grouped" if isinstance(cfg, synth.GroupedConfig) else "gemm"
    return [os.path.join(CSRC, f) for f in KERNEL_SOURCES[kind]]


def kernel_source_hash(cfg) -> str:
    """Hash of the kernel sources a workload runs, with comments and
    whitespace removed, so that edits of comments (or of other kernels) do
    not invalidate counters taken on the code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in _sources_for(cfg):
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_path(cfg) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{cfg.name}.json")


def stored_traffic(cfg):
    """HBM bytes per launch measured with rocprofv3 counters for this
    workload, if they were taken on the current kernel source; else None."""
    try:
        with open(traffic_path(cfg)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(cfg):
        return None
    return t.get("bytes_per_launch")


def _counter_per_dispatch(directory: str, counter: str, name_filter):
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or not name_filter(r["Kernel_Name"]):
                continue
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def traffic_summary(cfg, fetch_dir, write_dir, cfetch_dir, cwrite_dir, alg_bytes=None):
    nv_kernel = lambda n: "nvfp4" in n
    copy_kernel = lambda n: "nvfp4" not in n and ("copy" in n.lower() or "elementwise" in n.lower())
    f = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", nv_kernel)
    w = _counter_per_dispatch(write_dir, "WRITE_SIZE", nv_kernel)
    cf = _counter_per_dispatch(cfetch_dir, "FETCH_SIZE", copy_kernel)
    cw = _counter_per_dispatch(cwrite_dir, "WRITE_SIZE", copy_kernel)
    if not (f and w and cf and cw):
        raise SystemExit("missing counter records")
    # median dispatch of each; the copy moves COPY_BYTES each way
    med = lambda v: sorted(v)[len(v) // 2]
    kf, kw, ccf, ccw = med(f), med(w), med(cf), med(cw)
    scale_f = COPY_BYTES / (ccf * 1024.0)
    scale_w = COPY_BYTES / (ccw * 1024.0)
    fetch_b = kf * 1024.0 * scale_f
    write_b = kw * 1024.0 * scale_w
    out = {"workload": cfg.name, "M": cfg.M, "N": cfg.N, "K": cfg.K,
           "fetch_size_kib_per_dispatch": kf, "write_size_kib_per_dispatch": kw,
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": ccf, "copy_write_kib": ccw,
           "fetch_scale": scale_f, "write_scale": scale_w,
           "bytes_per_launch": fetch_b + write_b,
           "algorithmic_bytes_per_launch": (alg_bytes if alg_bytes is not None
                                            else synth.algorithmic_bytes(cfg.M, cfg.N, cfg.K)),
           "kernel_source_sha256_16": kernel_source_hash(cfg)}
    with open(traffic_path(cfg), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def copy_calibration(steps):
    import torch
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(max(1, steps)):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "calls": max(1, steps)}))


def path_name(nv, path: int) -> str:
    return {nv.PATH_SKINNY: "skinny", nv.PATH_WSPLIT: "wsplit", nv.PATH_TILE: "tile",
            nv.PATH_GEMV: "gemv"}.get(path, str(path))


def _roofline(b, f, seconds_per_call):
    """The binding roofline (HBM below the ridge AI = 2.5 PF / 8 TB/s, else
    the fp16 MFMA peak), with the other resource's rate beside it."""
    gbps = b / seconds_per_call / 1e9
    tflops = f / seconds_per_call / 1e12
    hbm = {"achieved": gbps, "peak": HBM_GBPS, "unit": "GB/s", "frac": gbps / HBM_GBPS}
    mfma = {"achieved": tflops, "peak": MFMA_F16_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / MFMA_F16_TFLOPS}
    if f / b < MFMA_F16_TFLOPS * 1e12 / (HBM_GBPS * 1e9):
        return {"bound": "hbm", **hbm, "traffic": None, "algorithmic_bytes_per_launch": b,
                "algorithmic_flops_per_launch": f, "other": dict(resource="mfma", **mfma)}
    return {"bound": "mfma", **mfma, "traffic": None, "algorithmic_flops_per_launch": f,
            "algorithmic_bytes_per_launch": b, "other": dict(resource="hbm", **hbm)}


def roofline_for(cfg, seconds_per_call):
    return _roofline(synth.algorithmic_bytes(cfg.M, cfg.N, cfg.K),
                     synth.flops(cfg.M, cfg.N, cfg.K), seconds_per_call)


def _operand_sets(nv, torch, cfg, ops, cold):
    a = nv.to_device(ops.a_codes, ops.a_scales, "cuda")
    b = nv.to_device(ops.b_codes, ops.b_scales, "cuda")
    out = torch.empty((cfg.M, cfg.N), dtype=torch.bfloat16, device="cuda")
    if not cold:
        return [(a, b, out)]
    # distinct operand copies whose total exceeds the 256 MB last-level cache twice
    per = a.codes.numel() + a.scales.numel() + b.codes.numel() + b.scales.numel()
    n = max(2, min(2048, int(2 * 256e6 // per) + 1))
    return [(nv.PackedOperand(a.codes.clone(), a.scales.clone(), a.rows, a.K),
             nv.PackedOperand(b.codes.clone(), b.scales.clone(), b.rows, b.K),
             torch.empty_like(out)) for _ in range(n)]


WARM_MS = 50.0          # device time a captured graph replays before its timed replay
MAX_WARM_REPLAYS = 2000


def timed_replay(torch, gr, stream, calls, warm_ms=WARM_MS):
    """Per-call device time of the captured graph `gr` (holding `calls`
    calls), measured on a warm GPU with the host ahead of the device.

    One replay sizes the warm-up; after a synchronisation, replays making
    about `warm_ms` of device time (two at least) and then the timed replay,
    between two HIP events on `stream`, are enqueued back to back, and the
    device is synchronised again.  Two effects are kept out of the figure:
    * the first replays after a capture or an idle gap run slow (the grouped
      GEMM's graph of 50 calls: 56, 52, 50 us per call in replays 2-4, about
      43 us from the tenth on; an empty kernel's first replay after 1 s idle:
      7.4 us per call against 1.76);
    * the host can take longer to enqueue a graph than the device takes to
      run it (50 decode-sized calls: 40-70 us to enqueue as a rule, up to
      600 us right after a long backlog drained), so a timed replay enqueued
      onto an idle device would time the host.
    Returns (ms per call of the timed replay, warm replays, wall seconds from
    the first warm replay to the end of the timed one)."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        gr.replay()
        stop.record(stream)
    stop.synchronize()
    first = max(start.elapsed_time(stop), 1e-3)
    more = int(min(MAX_WARM_REPLAYS - 1, max(1, -(-(warm_ms - first) // first))))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for _ in range(more):
            gr.replay()
        start.record(stream)
        gr.replay()
        stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / calls, 1 + more, wall


def time_workload(nv, torch, cfg, steps, warmup, cold=False, ops=None):
    """Per-call time of nvfp4_gemm on resident operands.

    'graph': the `steps` calls are captured once into a HIP graph (no memset
    or allocation inside: the split-K workspace exists after the warm-up),
    warmed by replays and replayed once more between two events
    (timed_replay), so the figure is the device time per call without host
    launch overhead.  'eager': the same calls
    issued one by one from Python between two events (host overhead
    included when the host is slower than the device)."""
    if ops is None:
        ops = synth.make_inputs(cfg)
    sets = _operand_sets(nv, torch, cfg, ops, cold)
    if cold:
        # every copy once per replay, so that each timed call reads operands
        # last touched more than twice the last-level cache's size ago
        steps = max(steps, len(sets))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(max(1, warmup)):
            x, y, o = sets[i % len(sets)]
            nv.gemm(x, y, cfg.alpha, out=o, stream=stream)
    stream.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    # eager
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        start.record(stream)
        for i in range(steps):
            x, y, o = sets[i % len(sets)]
            nv.gemm(x, y, cfg.alpha, out=o, stream=stream)
        stop.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(stop) / steps
    # graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        cap = torch.cuda.current_stream()
        for i in range(steps):
            x, y, o = sets[i % len(sets)]
            nv.gemm(x, y, cfg.alpha, out=o, stream=cap)
    graph_ms, warm_replays, wall = timed_replay(torch, g, stream, steps)
    plan = nv.plan(cfg.M, cfg.N, cfg.K)
    # the timed replay's own output (warm: every call wrote the one output
    # buffer), copied out after the timing for the parity check
    out_bits = None if cold else sets[0][2].view(torch.int16).cpu().numpy().astype(np.uint16)
    copies = len(sets)
    del g, sets
    return {"graph_ms": graph_ms, "eager_ms": eager_ms, "wall_s": wall, "plan": plan, "ops": ops,
            "out_bits": out_bits, "warm_replays": warm_replays, "calls_per_replay": steps,
            "operand_copies": copies}


def grouped_roofline(g, seconds_per_call):
    """As roofline_for, with the grouped GEMM's algorithmic bytes (A, the
    weights of every expert, the output)."""
    return _roofline(synth.grouped_algorithmic_bytes(g.M, g.N, g.K, g.experts),
                     synth.flops(g.M, g.N, g.K), seconds_per_call)


def time_grouped(nv, torch, g, steps, warmup, ops=None, cold=False):
    """Per-call time of nvfp4_grouped_gemm (all experts of one layer in one
    launch) on resident operands, graph-replayed like time_workload.  cold:
    the calls rotate over copies of A and of the weights whose total exceeds
    twice the 256 MB last-level cache (every copy once per replay), so each
    call reads its operands from HBM."""
    if ops is None:
        ops = synth.make_grouped_inputs(g)
    a = nv.to_device(ops.a_codes, ops.a_scales, "cuda")
    b = nv.groups_to_device(ops.b_codes, ops.b_scales, "cuda")
    off = torch.from_numpy(ops.offsets).to("cuda")
    out = torch.empty((ops.M, ops.N), dtype=torch.bfloat16, device="cuda")
    sets = [(a, b, out)]
    if cold:
        per = a.codes.numel() + a.scales.numel() + b.codes.numel() + b.scales.numel()
        n = max(2, int(2 * 256e6 // per) + 1)
        sets = [(nv.PackedOperand(a.codes.clone(), a.scales.clone(), a.rows, a.K),
                 nv.PackedGroups(b.codes.clone(), b.scales.clone(), b.groups, b.rows, b.K),
                 torch.empty_like(out)) for _ in range(n)]
        steps = max(steps, n)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(max(1, warmup)):
            x, y, o = sets[i % len(sets)]
            nv.grouped_gemm(x, y, off, g.alpha, out=o, stream=stream)
    stream.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=stream):
        cap = torch.cuda.current_stream()
        for i in range(steps):
            x, y, o = sets[i % len(sets)]
            nv.grouped_gemm(x, y, off, g.alpha, out=o, stream=cap)
    ms, warm_replays, _ = timed_replay(torch, gr, stream, steps)
    copies = len(sets)
    # the timed replay's own output (warm), for the parity check after the timing
    out_bits = None if cold else sets[0][2].view(torch.int16).cpu().numpy().astype(np.uint16)
    del gr, sets
    return {"graph_ms": ms, "ops": ops, "warm_replays": warm_replays, "calls_per_replay": steps,
            "operand_copies": copies, "out_bits": out_bits}


def grouped_line(nv, torch, steps, warmup, g=None):
    """One grouped workload (the decode batch by default), warm and cold;
    the library picks the kernel from the rows per expert.  Returns the
    workload's name, its line, and (config, operands, the warm run's output
    bits) for the parity check."""
    g = synth.GROUPED_CONFIGS[0] if g is None else g
    r = time_grouped(nv, torch, g, steps, warmup)
    ms = r["graph_ms"]
    c = time_grouped(nv, torch, g, steps, warmup, ops=r["ops"], cold=True)
    cms = c["graph_ms"]
    counts = np.diff(r["ops"].offsets)
    return g.name, {"experts": g.experts, "tokens": g.tokens, "top_k": g.top_k, "M": g.M,
                    "N": g.N, "K": g.K, "rows_per_expert": [int(counts.min()), int(counts.max())],
                    "ms": ms, "tflops": synth.flops(g.M, g.N, g.K) / (ms * 1e-3) / 1e12,
                    "roofline": dict(grouped_roofline(g, ms * 1e-3), traffic=stored_traffic(g)),
                    "cold": {"ms": cms, "tflops": synth.flops(g.M, g.N, g.K) / (cms * 1e-3) / 1e12,
                             "roofline": grouped_roofline(g, cms * 1e-3),
                             "operand_copies": c["operand_copies"],
                             "calls_per_replay": c["calls_per_replay"],
                             "note": "operand copies rotated beyond the last-level cache"},
                    "path": "grouped (kernel chosen from the rows per expert)",
                    "pages_tflops_other_gpu": None}, (g, r["ops"], r["out_bits"])


QUANT_SHAPES = [(16, 6144), (16384, 8192)]   # decode activations of one expert; saturation-shape A


def quantize_bytes(rows: int, K: int, in_bytes: int = 4) -> int:
    """Input read once (4 bytes per fp32 value, 2 per bfloat16) plus the
    packed output written (padding included)."""
    rp = -(-rows // 16) * 16
    kp = -(-K // 128) * 128
    return rows * K * in_bytes + rp * kp // 2 + rp * kp // 16


def quantize_line(nv, torch, rows, K, steps, warmup, bf16=False):
    """Per-call time of nvfp4_quantize (nvfp4_quantize_bf16) on a resident
    fp32 (bfloat16) tensor, graph-replayed."""
    g = np.random.Generator(np.random.PCG64(rows + K))
    x = torch.from_numpy(g.standard_normal((rows, K), dtype=np.float32)).to("cuda")
    if bf16:
        x = x.to(torch.bfloat16)
    out = nv.quantize(x)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup)):
            nv.quantize(x, out=out, stream=stream)
    stream.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=stream):
        cap = torch.cuda.current_stream()
        for _ in range(steps):
            nv.quantize(x, out=out, stream=cap)
    ms, _, _ = timed_replay(torch, gr, stream, steps)
    b = quantize_bytes(rows, K, 2 if bf16 else 4)
    ach = b / (ms * 1e-3) / 1e9
    del gr
    return f"quantize_{'bf16_' if bf16 else ''}{rows}x{K}", {
        "rows": rows, "K": K, "input": "bfloat16" if bf16 else "float32", "ms": ms,
        "gelem_per_s": rows * K / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_GBPS, "unit": "GB/s",
                     "frac": ach / HBM_GBPS, "traffic": None, "algorithmic_bytes_per_launch": b},
        "path": "quantize"}


DECODE_LAYERS = 8


def decode_sequence_line(nv, torch, steps, warmup):
    """A decode step of DECODE_LAYERS layers, each quantising the fp32
    activations and running the attention projection (1 x 768 x 6144) and
    the MoE up-projection share (16 x 256 x 6144) with its own weights:
    4 calls per layer.  Timed as eager calls from Python (host launch gaps
    included: the device waits for them) and as one recorded sequence
    (nvfp4_sequence_launch) per step, both between HIP events."""
    K = 6144
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(2026)
    x1 = torch.randn((1, K), generator=g, device=dev)
    x16 = torch.randn((16, K), generator=g, device=dev)
    a1 = nv.quantize(x1)
    a16 = nv.quantize(x16)
    layers = []
    for _ in range(DECODE_LAYERS):
        w_attn = nv.quantize(torch.randn((768, K), generator=g, device=dev) * 0.02)
        w_up = nv.quantize(torch.randn((256, K), generator=g, device=dev) * 0.02)
        layers.append((w_attn, w_up, torch.empty((1, 768), dtype=torch.bfloat16, device=dev),
                       torch.empty((16, 256), dtype=torch.bfloat16, device=dev)))
    stream = torch.cuda.Stream()

    def eager_step():
        for w_attn, w_up, o1, o16 in layers:
            nv.quantize(x1, out=a1, stream=stream)
            nv.gemm(a1, w_attn, 0.5, out=o1, stream=stream)
            nv.quantize(x16, out=a16, stream=stream)
            nv.gemm(a16, w_up, 1.0, out=o16, stream=stream)

    seq = nv.Sequence()
    for w_attn, w_up, o1, o16 in layers:
        seq.add_quantize(x1, a1)
        seq.add_gemm(a1, w_attn, o1, 0.5)
        seq.add_quantize(x16, a16)
        seq.add_gemm(a16, w_up, o16, 1.0)
    seq.finalize()
    # the same step with the one-row projection quantising its own
    # activations (nvfp4_gemm_quantized): 3 calls per layer
    seq_f = nv.Sequence()
    for w_attn, w_up, o1, o16 in layers:
        seq_f.add_gemm_quantized(x1, w_attn, 0.5, o1)
        seq_f.add_quantize(x16, a16)
        seq_f.add_gemm(a16, w_up, o16, 1.0)
    seq_f.finalize()

    def timed(fn):
        # warm-up as in timed_replay: `warmup` steps, then as many more as
        # make about WARM_MS of device time, with the timed steps enqueued
        # right behind them (a warm GPU, and the host ahead of the device
        # when the timed region starts)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            start.record(stream)
            for _ in range(max(1, warmup)):
                fn()
            stop.record(stream)
        stop.synchronize()
        per = max(start.elapsed_time(stop) / max(1, warmup), 1e-3)
        with torch.cuda.stream(stream):
            for _ in range(int(min(MAX_WARM_REPLAYS, max(1, WARM_MS // per)))):
                fn()
            start.record(stream)
            for _ in range(steps):
                fn()
            stop.record(stream)
        stop.synchronize()
        return start.elapsed_time(stop) * 1000.0 / steps   # us per step

    eager_us = timed(eager_step)
    seq_us = timed(lambda: seq.launch(stream))
    fused_us = timed(lambda: seq_f.launch(stream))
    calls, calls_f = seq.calls, seq_f.calls
    seq.close()
    seq_f.close()
    return "decode_step_sequence", {
        "layers": DECODE_LAYERS, "calls_per_step": calls,
        "calls": "per layer: quantize 1x6144, GEMM 1x768x6144, quantize 16x6144, GEMM 16x256x6144",
        "us_per_step_eager": eager_us, "us_per_step_sequence": seq_us,
        "us_per_call_eager": eager_us / calls, "us_per_call_sequence": seq_us / calls,
        "speedup": eager_us / seq_us,
        "fused_calls_per_step": calls_f,
        "fused_calls": "per layer: GEMM 1x768x6144 quantising its fp32 row (nvfp4_gemm_quantized), "
                       "quantize 16x6144, GEMM 16x256x6144",
        "us_per_step_sequence_fused": fused_us,
        "path": "sequence (one HIP graph launch per step)"}


def fused_projection_line(nv, torch, steps, warmup):
    """The decode attention projection from unquantised activations (one
    row of 6144, N = 768, alpha 0.5), per call in a graph replay: quantise
    then GEMM (two launches) against nvfp4_gemm_quantized (one), for fp32
    and bfloat16 rows; the outputs of the two forms are compared bit for bit."""
    K, N = 6144, 768
    g = torch.Generator(device="cuda").manual_seed(2027)
    b = nv.quantize(torch.randn((N, K), generator=g, device="cuda") * 0.02)
    res = {"shape": "1 x 768 x 6144", "alpha": 0.5}
    for name, dt in (("float32", torch.float32), ("bfloat16", torch.bfloat16)):
        x = torch.randn((1, K), generator=g, device="cuda").to(dt)
        a = nv.quantize(x)
        o2 = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")
        o1 = torch.empty_like(o2)
        stream = torch.cuda.Stream()

        def per_call(fn):
            with torch.cuda.stream(stream):
                for _ in range(max(1, warmup)):
                    fn(stream)
            stream.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=stream):
                cap = torch.cuda.current_stream()
                for _ in range(steps):
                    fn(cap)
            ms, _, _ = timed_replay(torch, gr, stream, steps)
            del gr
            return ms * 1000.0

        two = per_call(lambda s: (nv.quantize(x, out=a, stream=s), nv.gemm(a, b, 0.5, out=o2, stream=s)))
        one = per_call(lambda s: nv.gemm_quantized(x, b, 0.5, out=o1, stream=s))
        res[name] = {"us_quantize_then_gemm": two, "us_gemm_quantized": one,
                     "identical": bool(torch.equal(o1.view(torch.int16), o2.view(torch.int16)))}
    return "decode_attn_proj_from_activations", res


def floors_line(nv, torch, steps):
    """The floors under the decode-sized calls, measured on this GPU: the
    per-call time of an empty kernel with the headline's launch shape (768/4
    workgroups of 256 work-items) in a graph replay, timed like the GEMMs,
    and the latency of one dependent load when the data sit in one XCD's L2,
    in the last-level cache, or only in HBM (one work-item walking a random
    single cycle through 1 MiB, 64 MiB or 1 GiB)."""
    stream = torch.cuda.Stream()
    blocks, threads = 768 // 4, 256
    with torch.cuda.stream(stream):
        for _ in range(3):
            nv.probe_empty(blocks, threads, stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        cap = torch.cuda.current_stream()
        for _ in range(steps):
            nv.probe_empty(blocks, threads, stream=cap)
    empty_ms, _, _ = timed_replay(torch, g, stream, steps)
    empty_us = empty_ms * 1000.0
    del g
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    lat = {}
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    # HBM first, on a buffer no load has touched (4x the last-level cache);
    # then 64 MiB after one read of it (the last-level cache holds it); then
    # 1 MiB after one full walk on the same single work-item (its XCD's L2
    # holds it).  Every walk starts at index 0 and its last index is checked
    # against the same walk on the host.
    for name, size, walk in (("hbm_1GiB", 1 << 30, 5000), ("last_level_64MiB", 64 << 20, 5000),
                             ("l2_1MiB", 1 << 20, 5000)):
        n = size // 4
        perm = torch.randperm(n, device="cuda")
        nxt = torch.empty(n, dtype=torch.int32, device="cuda")
        nxt[perm] = torch.roll(perm, -1).to(torch.int32)   # one cycle through all n entries
        del perm
        host = nxt.cpu().numpy()
        i = 0
        for _ in range(walk):
            i = int(host[i])
        del host
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            if name.startswith("l2"):
                nv.probe_chase(nxt, n, out, stream=stream)   # one full pass, back to index 0
            elif name.startswith("last_level"):
                nxt.sum()
            start.record(stream)
            nv.probe_chase(nxt, walk, out, stream=stream)
            stop.record(stream)
        torch.cuda.synchronize()
        if int(out.item()) != i:
            raise RuntimeError(f"pointer chase over {name} ended at {int(out.item())}, expected {i}")
        lat[name] = start.elapsed_time(stop) * 1e6 / walk
        del nxt
        torch.cuda.empty_cache()
    return {"empty_kernel_us_per_call": empty_us,
            "empty_kernel_launch": f"{blocks} workgroups of {threads} work-items, graph replay of {steps}",
            "load_latency_ns": lat,
            "load_latency_how": "one work-item, dependent loads along a random cycle"}


def measured_peaks(nv, torch, steps):
    """The two peaks measured on this GPU with the library's measurement aids:
    the fp16 MFMA rate (nvfp4_probe_mfma: 1024 workgroups x 4 waves, 8
    independent 32 x 32 x 16 MFMAs per round) and the rate of a streaming
    read of 1 GiB from HBM (nvfp4_probe_read, 16-byte loads; best of two grid
    sizes), each timed over a graph replay of several launches."""
    stream = torch.cuda.Stream()

    def replay_ms(fn, reps):
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                fn()
        ms, _, _ = timed_replay(torch, g, stream, reps)
        del g
        return ms

    blocks, iters = 1024, 2000
    mout = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ms = replay_ms(lambda: nv.probe_mfma(blocks, iters, mout, stream=torch.cuda.current_stream()), 5)
    mfma = blocks * 4 * iters * 8 * 2 * 32 * 32 * 16 / (ms * 1e-3) / 1e12
    del mout
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src.random_(0, 256)
    rout = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = 0.0
    for b in (2048, 8192):
        rms = replay_ms(lambda: nv.probe_read(src, b, rout, stream=torch.cuda.current_stream()), 5)
        best = max(best, src.numel() / (rms * 1e-3) / 1e9)
    del src
    torch.cuda.empty_cache()
    return {"mfma_f16_tflops": mfma, "hbm_read_gbps": best,
            "how": "nvfp4_probe_mfma (1024 x 4 waves x 2000 rounds of 8 fp16 32x32x16 MFMAs) and "
                   "nvfp4_probe_read (1 GiB, best of 2048 / 8192 workgroups), graph replays of 5"}


def add_measured_fracs(node, peaks):
    """Every roofline object in the line (and the other resource beside it)
    also gets its fraction of the measured peak of that resource."""
    if isinstance(node, dict):
        kind = node.get("bound", node.get("resource"))
        if kind in ("hbm", "mfma") and "achieved" in node:
            p = peaks["hbm_read_gbps"] if kind == "hbm" else peaks["mfma_f16_tflops"]
            node["peak_measured"] = p
            node["frac_of_measured"] = node["achieved"] / p
        for v in node.values():
            add_measured_fracs(v, peaks)


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def oracle_leg(o, cfg, ops, gpu_bits):
    """Parity of the timed run's output against the oracle, and the oracle's
    own time for it (all host threads).  Full matrix up to 10^10 MACs; above
    that, whole rows, columns, tiles and random elements (oracle/parity.py's
    large_sample), with the full-matrix oracle time extrapolated by MACs."""
    from oracle import parity
    M, N, K = cfg.M, cfg.N, cfg.K
    if M * N * K <= 10 ** 10:
        t0 = time.perf_counter()
        bits, exact, mag = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, cfg.alpha)
        el = time.perf_counter() - t0
        r = parity.compare(gpu_bits, bits, exact, mag, cfg.alpha)
        return ({k: r[k] for k in ("n", "over", "max_err_over_tol", "bit_exact_frac")} |
                {"elements": "all"},
                {"oracle_s": el, "tflops": synth.flops(M, N, K) / el / 1e12, "threads": o.threads,
                 "sample": "the full GEMM once"})
    sample = parity.large_sample(M, N)
    r = parity.check_sample(o, ops, gpu_bits, sample)
    macs = r["n"] * K
    el = r["oracle_s"]
    what = (f"rows {sample['rows']}, columns {sample['cols']}, {len(sample['tiles'])} whole 256x256 "
            f"tiles at {sample['tiles']}, {len(sample['points'][0])} random elements")
    return ({k: r[k] for k in ("n", "over", "max_err_over_tol", "bit_exact_frac")} |
            {"elements": what},
            {"oracle_s": el, "tflops": 2 * macs / el / 1e12, "threads": o.threads,
             "full_matrix_s_extrapolated": el * (M * N * K) / macs,
             "sample": f"{r['n']} output elements ({what}); the full-matrix time is extrapolated "
                       "by the number of multiply-adds"})


def grouped_oracle_leg(o, g, ops, gpu_bits):
    """Parity of a timed grouped run's output against the oracle (each
    expert's rows an ordinary GEMM with that expert's weights), and the
    oracle's time: every expert up to 10^11 multiply-adds (a few seconds on
    16 host threads); above that 16
    whole experts (the first, the last, the smallest and the largest
    non-empty ones, 12 more drawn with a fixed seed), the oracle's time for
    the whole layer extrapolated by multiply-adds."""
    from oracle import parity
    counts = np.diff(ops.offsets)
    nonempty = [int(e) for e in np.flatnonzero(counts)]
    if g.M * g.N * g.K <= 10 ** 11:
        experts, what = nonempty, "every expert"
    else:
        rng = np.random.Generator(np.random.PCG64(g.M))
        pick = {nonempty[0], nonempty[-1], min(nonempty, key=lambda e: counts[e]),
                max(nonempty, key=lambda e: counts[e])}
        rest = [e for e in nonempty if e not in pick]
        pick |= {int(e) for e in rng.choice(rest, size=min(12, len(rest)), replace=False)}
        experts = sorted(pick)
        what = f"{len(experts)} whole experts {experts}"
    reports, macs = [], 0
    t0 = time.perf_counter()
    for e in experts:
        r0, r1 = int(ops.offsets[e]), int(ops.offsets[e + 1])
        bits, exact, mag = o.gemm(np.ascontiguousarray(ops.a_codes[r0:r1]),
                                  np.ascontiguousarray(ops.a_scales[r0:r1]), ops.b_codes[e],
                                  ops.b_scales[e], g.alpha)
        reports.append(parity.compare(gpu_bits[r0:r1], bits, exact, mag, g.alpha))
        macs += (r1 - r0) * g.N * g.K
    el = time.perf_counter() - t0
    r = parity.merge(reports)
    return ({k: r[k] for k in ("n", "over", "max_err_over_tol", "bit_exact_frac")} |
            {"elements": what},
            {"oracle_s": el, "tflops": 2 * macs / el / 1e12, "threads": o.threads,
             "full_layer_s_extrapolated": el * (g.M * g.N * g.K) / macs,
             "sample": f"{r['n']} output elements ({what})"})


def host_pack_ms(nv, ops, reps=3):
    """Host time of packing A's canonical arrays (nvfp4_pack, one thread),
    best of `reps`; B is packed once, as weights, and not timed."""
    best = float("inf")
    for _ in range(reps):
        t0 = time.perf_counter()
        nv.pack(ops.a_codes, ops.a_scales)
        best = min(best, time.perf_counter() - t0)
    return best * 1e3


def cpu_baseline(cfg, ops, budget_s):
    from oracle import oracle as orc
    o = orc.load()
    # one call first to size the sample
    t0 = time.perf_counter()
    o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, cfg.alpha, want_exact=False)
    one = time.perf_counter() - t0
    reps = max(1, int(budget_s / max(one, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, cfg.alpha, want_exact=False)
    el = time.perf_counter() - t0
    tflops = synth.flops(cfg.M, cfg.N, cfg.K) * reps / el / 1e12
    # the oracle spreads its output elements over all its OpenMP threads
    return {"value": tflops, "unit": "TFLOPS", "cores": min(o.threads, cfg.M * cfg.N),
            "kind": "oracle",
            "sample": f"the full {cfg.M}x{cfg.N}x{cfg.K} GEMM repeated {reps} times "
                      f"({el:.1f} s, fp64 C oracle, OpenMP over output elements)"}


def main():
    args = parse()
    if args.traffic_summary:
        if args.grouped_only:
            g = synth.grouped_config(args.grouped_workload)
            traffic_summary(g, *args.traffic_summary,
                            alg_bytes=synth.grouped_algorithmic_bytes(g.M, g.N, g.K, g.experts))
        else:
            traffic_summary(synth.config(args.workload), *args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the GEMM's "
              "multi-GPU sharding is described in the design notes but not built.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_fp4_04_amd as nv
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    nv.init(torch.cuda.current_device())
    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    if args.quantize_only:
        for bf16 in (False, True):
            for rows, K in QUANT_SHAPES:
                name, q = quantize_line(nv, torch, rows, K, args.steps, args.warmup, bf16)
                print(json.dumps({"workload": name, **q}), flush=True)
        return
    if args.decode_only:
        name, d = decode_sequence_line(nv, torch, args.steps, args.warmup)
        print(json.dumps({"workload": name, **d}), flush=True)
        name, d = fused_projection_line(nv, torch, args.steps, args.warmup)
        print(json.dumps({"workload": name, **d}), flush=True)
        return
    if args.grouped_only:
        name, g, _ = grouped_line(nv, torch, args.steps, args.warmup,
                                  synth.grouped_config(args.grouped_workload))
        print(json.dumps({"workload": name, **g}), flush=True)
        return
    if args.floors_only:
        f = floors_line(nv, torch, args.steps)
        f["measured_peaks"] = measured_peaks(nv, torch, args.steps)
        print(json.dumps({"floors": f}), flush=True)
        return
    peaks = None if args.only_headline else measured_peaks(nv, torch, args.steps)

    cfg = synth.config(args.workload)
    r = time_workload(nv, torch, cfg, args.steps, args.warmup)
    ms, plan, ops = r["graph_ms"], r["plan"], r["ops"]
    outputs = {cfg.name: (cfg, ops, r["out_bits"])}   # checked against the oracle at the end
    grouped_outputs = {}
    tflops = synth.flops(cfg.M, cfg.N, cfg.K) / (ms * 1e-3) / 1e12
    line = {
        "metric": "NVFP4 GEMM TFLOPS (2MNK/s) per shape + % of HBM/MFMA roofline, 1 MI355X",
        "value": tflops, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (tflops / PAGES_TFLOPS[cfg.index]) if PAGES_TFLOPS.get(cfg.index) else None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} M={cfg.M} N={cfg.N} K={cfg.K} alpha={cfg.alpha}",
                   "M": cfg.M, "N": cfg.N, "K": cfg.K, "alpha": cfg.alpha,
                   "path": path_name(nv, plan["path"]),
                   "split_k": plan["split_k"], "tile": [plan["tile_m"], plan["tile_n"]],
                   "operands": "E2M1 codes + E4M3 per-16 scales (packed), bf16 out, "
                               "fp16 MFMA with fp32 accumulation",
                   "timing": "HIP graph of the timed calls, replayed for about "
                             f"{WARM_MS:g} ms of device time and then once more between HIP "
                             "events, enqueued behind the warm replays",
                   "parallelism": "none (1 GPU)"},
        "roofline": dict(roofline_for(cfg, ms * 1e-3), traffic=stored_traffic(cfg)),
        "eager_ms_per_step": r["eager_ms"],
        "warm_replays": r["warm_replays"],
        "wall_s_warm_and_timed_replays": r["wall_s"],
    }
    if args.cold or not args.only_headline:
        c = time_workload(nv, torch, cfg, args.steps, args.warmup, cold=True, ops=ops)
        line["cold"] = {"ms_per_step": c["graph_ms"],
                        "tflops": synth.flops(cfg.M, cfg.N, cfg.K) / (c["graph_ms"] * 1e-3) / 1e12,
                        "roofline": roofline_for(cfg, c["graph_ms"] * 1e-3),
                        "operand_copies": c["operand_copies"],
                        "calls_per_replay": c["calls_per_replay"],
                        "note": "operand copies rotated beyond the last-level cache"}
    if not args.only_headline:
        per = {}
        # the grouped workloads first, then the single GEMMs by size; the
        # allocator's cached blocks are released between workloads
        torch.cuda.empty_cache()
        for gc in synth.GROUPED_CONFIGS:
            name, g, grouped_outputs[name] = grouped_line(nv, torch, args.steps, args.warmup, gc)
            per[name] = g
            torch.cuda.empty_cache()
        name, d = decode_sequence_line(nv, torch, args.steps, args.warmup)
        per[name] = d
        name, d = fused_projection_line(nv, torch, args.steps, args.warmup)
        per[name] = d
        for bf16 in (False, True):
            for rows, K in QUANT_SHAPES:
                torch.cuda.empty_cache()
                name, q = quantize_line(nv, torch, rows, K, args.steps, args.warmup, bf16)
                per[name] = q
        for c in synth.CONFIGS:
            if c.index == cfg.index:
                continue
            torch.cuda.empty_cache()
            cr = time_workload(nv, torch, c, args.steps, args.warmup)
            cms = cr["graph_ms"]
            ctf = synth.flops(c.M, c.N, c.K) / (cms * 1e-3) / 1e12
            outputs[c.name] = (c, cr["ops"], cr["out_bits"])
            per[c.name] = {"M": c.M, "N": c.N, "K": c.K, "ms": cms, "tflops": ctf,
                           "eager_ms": cr["eager_ms"],
                           "roofline": dict(roofline_for(c, cms * 1e-3), traffic=stored_traffic(c)),
                           "path": path_name(nv, cr["plan"]["path"]),
                           "split_k": cr["plan"]["split_k"],
                           "pages_tflops_other_gpu": PAGES_TFLOPS.get(c.index)}
            if c.M <= 16:   # the other decode-sized workload: also with operands beyond the cache
                cc = time_workload(nv, torch, c, args.steps, args.warmup, cold=True, ops=cr["ops"])
                per[c.name]["cold"] = {
                    "ms": cc["graph_ms"],
                    "tflops": synth.flops(c.M, c.N, c.K) / (cc["graph_ms"] * 1e-3) / 1e12,
                    "roofline": roofline_for(c, cc["graph_ms"] * 1e-3),
                    "operand_copies": cc["operand_copies"],
                    "calls_per_replay": cc["calls_per_replay"],
                    "note": "operand copies rotated beyond the last-level cache"}
        line["per_shape"] = per
        torch.cuda.empty_cache()
        line["floors"] = floors_line(nv, torch, args.steps)
        line["floors"]["measured_peaks"] = peaks
        add_measured_fracs(line, peaks)
    # after the GPU timing: the host time of packing each workload's A
    for name, (c, c_ops, _) in outputs.items():
        pack_ms = host_pack_ms(nv, c_ops)
        (line if c.index == cfg.index else line["per_shape"][name])["a_host_pack_ms"] = pack_ms
    if not args.no_cpu_baseline:
        # after every GPU timing: the oracle on all host threads, for the
        # headline's baseline figure and, per workload, for the parity of the
        # timed run's own output and the oracle's time
        from oracle import oracle as orc
        o = orc.load()
        cb = cpu_baseline(cfg, ops, args.cpu_seconds)
        cb["host"] = host_info() | {"oracle_threads": o.threads}
        cb["per_config"] = {}
        for name, (c, c_ops, bits) in outputs.items():
            par, stats = oracle_leg(o, c, c_ops, bits)
            cb["per_config"][name] = stats
            if c.index == cfg.index:
                line["parity"] = par
            else:
                line["per_shape"][name]["parity"] = par
        for name, (g, g_ops, bits) in grouped_outputs.items():
            par, stats = grouped_oracle_leg(o, g, g_ops, bits)
            cb["per_config"][name] = stats
            line["per_shape"][name]["parity"] = par
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
