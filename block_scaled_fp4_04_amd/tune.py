"""Offline sweep that writes the tuned plan table of the NVFP4 GEMM.

    python -m block_scaled_fp4_04_amd.tune [--out plan_table_gfx950.json] [--quick]

For each shape it times the library's own plan and a set of candidate plans
(kernel path, output tile, split-K) through nvfp4_gemm_with_plan, and keeps
the fastest; the library's plan is kept unless another is at least 2% faster
(the run-to-run spread of these timings is about 1%).  Timing: the calls are
captured in a HIP graph, replayed for about WARM_MS of device time and then
three more times between HIP events, all enqueued back to back so that the
device never waits for the host (enqueueing a graph of short calls can take
longer than running it) and runs at the clock it keeps under load; the best
of the three timed replays is kept.

Operands are seeded N(0, 1) values quantised on the GPU by nvfp4_quantize
(the power-limited clock of the MFMA-bound shapes depends on the data, so
all-zero or constant operands would time too fast).  Needs an MI355X.

The shapes are the benchmark workloads, the pages' GEMM sweep ("Peeling the
Kernel Onion", section "The Results": 2048-8192 x 2048 x 6144 and 1024-4096 x
6144 x 6144), and powers of two in M for the weight shapes (N, K) of those
workloads, so that nearby M find an entry (the library uses the entry with
the same N and K and the smallest tuned M' >= M, if M' <= 2 M).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import block_scaled_fp4_04_amd as nv

WEIGHT_SHAPES = [(256, 6144), (768, 6144), (2048, 6144), (6144, 6144), (8192, 8192)]
M_SWEEP = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384]
EXTRA_SHAPES = [(1, 2048, 6144)]
KEEP_MARGIN = 0.02
SKINNY_MAX_SPLIT = 16  # the skinny kernel's last arrival fetches one split per wave (16 waves)
WARM_MS = 10.0         # device time of the warm replays before a plan's timed replays


def shapes(quick: bool) -> list[tuple[int, int, int]]:
    ms = [1, 16, 512, 4096] if quick else M_SWEEP
    out = [(M, N, K) for N, K in WEIGHT_SHAPES for M in ms] + EXTRA_SHAPES
    return sorted(set(out), key=lambda s: (s[1], s[2], s[0]))


def candidates(M: int, N: int, K: int) -> list[tuple[int, int, int]]:
    """(path, tile, split_k) plans worth timing for a shape."""
    def cdiv(a, b):
        return -(-a // b)
    steps = cdiv(K, 128)
    out = []
    if M <= 4:
        out.append((nv.PATH_GEMV, 0, 1))
    if M <= 64:
        groups = cdiv(N, 16)
        for s in (1, 2, 3, 4, 8, 16):
            # at least four 128-element K steps per workgroup
            if s <= min(SKINNY_MAX_SPLIT, max(1, steps // 4)) and groups * s <= 4096:
                out.append((nv.PATH_SKINNY, 0, s))
    if M > 4 or N > 4096:
        for tile, (bm, bn) in ((16, (32, 32)), (32, (64, 32)), (64, (64, 64)), (128, (128, 64))):
            tiles = cdiv(M, bm) * cdiv(N, bn)
            for s in (1, 2, 3, 4, 6, 8):
                if s * 8 <= 2 * steps and tiles * s <= 2048 and (s == 1 or tiles * s <= 1024):
                    out.append((nv.PATH_WSPLIT, tile, s))
    if M > 16:
        for tile in (64, 128, 256):
            if tile > 64 and (M < tile // 2 or N < tile // 2):
                continue
            tiles = cdiv(M, tile) * cdiv(N, tile)
            for s in (1, 2, 3, 4, 8):
                if s * 2 <= steps and (s == 1 or tiles * s <= 1024):
                    out.append((nv.PATH_TILE, tile, s))
    return out


def make_operand(rows: int, K: int, seed: int, device):
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    x = torch.randn((rows, K), generator=g, device=device, dtype=torch.float32)
    q = nv.quantize(x)
    del x
    return q


def time_plan(a, b, out, plan, stream, reps: int) -> float:
    """Device microseconds per call of one plan (best of three timed
    replays behind about WARM_MS of warm replays)."""
    import torch
    path, tile, split = plan
    with torch.cuda.stream(stream):
        for _ in range(2):  # creates any split-K workspace outside the capture
            nv.gemm(a, b, 1.0, out=out, path=path, tile=tile, split_k=split, stream=stream)
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(reps):
            nv.gemm(a, b, 1.0, out=out, path=path, tile=tile, split_k=split, stream=stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(4)]
    with torch.cuda.stream(stream):
        ev[0][0].record(stream)
        g.replay()
        ev[0][1].record(stream)
    ev[0][1].synchronize()
    first = max(ev[0][0].elapsed_time(ev[0][1]), 1e-3)
    warm = int(min(500, max(1, WARM_MS // first)))
    with torch.cuda.stream(stream):
        for _ in range(warm):
            g.replay()
        for e0, e1 in ev[1:]:
            e0.record(stream)
            g.replay()
            e1.record(stream)
    stream.synchronize()
    best = min(e0.elapsed_time(e1) for e0, e1 in ev[1:]) * 1000.0 / reps
    del g
    return best


def tune_shape(M, N, K, device, stream, log) -> dict:
    import torch
    a = make_operand(M, K, 11 + M, device)
    b = make_operand(N, K, 13 + N + K, device)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    nv.clear_plan_table()
    h = nv.plan(M, N, K)
    heur = (h["path"], h["tile"], h["split_k"])
    # calls per graph: about 2 ms of work, at least 5
    t1 = time_plan(a, b, out, heur, stream, 5)
    reps = int(min(200, max(5, 2000.0 / max(t1, 1e-3))))
    times = {heur: time_plan(a, b, out, heur, stream, reps)}
    for c in candidates(M, N, K):
        if c not in times:
            times[c] = time_plan(a, b, out, c, stream, reps)
    best = min(times, key=times.get)
    if times[best] > (1.0 - KEEP_MARGIN) * times[heur]:
        best = heur
    flops = 2.0 * M * N * K
    log(f"{M}x{N}x{K}: library {nv.PATH_NAMES[heur[0]]}/{heur[1]}/{heur[2]} "
        f"{times[heur]:.2f} us; chosen {nv.PATH_NAMES[best[0]]}/{best[1]}/{best[2]} "
        f"{times[best]:.2f} us ({flops / times[best] / 1e6:.1f} TFLOPS, "
        f"{len(times)} plans timed)")
    log("    " + ", ".join(f"{nv.PATH_NAMES[c[0]]}/{c[1]}/{c[2]} {t:.2f}"
                          for c, t in sorted(times.items(), key=lambda kv: kv[1])))
    del a, b, out
    return {"M": M, "N": N, "K": K, "path": nv.PATH_NAMES[best[0]], "tile": best[1],
            "split_k": best[2], "us": round(times[best], 3),
            "library_plan_us": round(times[heur], 3)}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", default=nv.PLAN_TABLE_PATH)
    ap.add_argument("--quick", action="store_true", help="a few M per weight shape")
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("tune: needs a GPU", file=sys.stderr)
        return 2
    device = torch.device("cuda", torch.cuda.current_device())
    name = torch.cuda.get_device_properties(device).gcnArchName.split(":")[0]
    if name != "gfx950":
        print(f"tune: needs a gfx950 GPU, found {name}", file=sys.stderr)
        return 2

    def log(msg):
        print(msg, flush=True)

    stream = torch.cuda.Stream(device)
    entries = []
    t0 = time.time()
    for M, N, K in shapes(args.quick):
        entries.append(tune_shape(M, N, K, device, stream, log))
        torch.cuda.empty_cache()
    doc = {"format": "nvfp4-plan-table", "version": 1, "arch": "gfx950",
           "build": nv.build_id(),
           "how": "device time per call in HIP graph replay, best of 3 behind "
                  f"{WARM_MS:g} ms of warm replays; operands N(0,1) quantised; library "
                  "plan kept unless another is 2% faster",
           "entries": entries}
    tmp = args.out + ".tmp"
    with open(tmp, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    os.replace(tmp, args.out)
    nv.load_default_plan_table()
    log(f"wrote {len(entries)} entries to {args.out} in {time.time() - t0:.0f} s")
    return 0


if __name__ == "__main__":
    sys.exit(main())
