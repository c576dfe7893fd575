"""The measurement model: algorithmic bytes and FLOPs.

Pinned by the size-sweep table of "Peeling the Kernel Onion" (section "The
Results"): its arithmetic-intensity column follows from the bytes formula of
section "The Benchmark Design" with 2*M*N*K operations.  Five printed values
are the formula rounded to an integer; the last (3,608) is 0.51 above the
formula's 3,607.49, so the check allows 0.6."""
import synth

# (M, N, K, printed AI) from the table
TABLE = [(2048, 2048, 6144, 2286), (4096, 2048, 6144, 2712), (8192, 2048, 6144, 2990),
         (1024, 6144, 6144, 2070), (2048, 6144, 6144, 2891), (4096, 6144, 6144, 3608)]


def test_ai_column_reproduces():
    for M, N, K, ai in TABLE:
        got = synth.flops(M, N, K) / synth.algorithmic_bytes(M, N, K)
        assert abs(got - ai) < 0.6, (M, N, K, got, ai)


def test_config_bytes():
    want = {1: 948224, 2: 2659200, 3: 5210112, 4: 10944512, 5: 381681664}
    for i, b in want.items():
        c = synth.config(i)
        assert synth.algorithmic_bytes(c.M, c.N, c.K) == b


def _grouped(seed, tokens, experts, N, K):
    ops = synth.grouped_operands(seed, tokens, experts, 4, N, K)
    cfg = synth.GroupedConfig("t", tokens, experts, 4, N, K, 1.0, seed, "test")
    return cfg, ops


def test_grouped_oracle_leg_checks_every_expert_or_a_sample():
    """The benchmark's grouped parity leg: on the oracle's own bits every
    checked element is exact; a one-element error in a checked expert is
    counted; above the size limit only 16 whole sampled experts are checked
    (the first, the last, the smallest, the largest and 12 drawn), and their
    rows are what is reported."""
    import ast
    import types

    import numpy as np

    import bench
    from oracle import oracle as orc
    o = orc.load()
    cfg, ops = _grouped(3, 40, 8, 24, 128)
    ref, _, _ = o.grouped_gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.offsets,
                               cfg.alpha)
    par, stats = bench.grouped_oracle_leg(o, cfg, ops, ref)
    assert par["over"] == 0 and par["bit_exact_frac"] == 1.0 and par["n"] == cfg.M * cfg.N
    assert par["elements"] == "every expert"
    bad = ref.copy()
    bad[int(ops.offsets[-1]) - 1, 5] ^= 0x4000           # flip an exponent bit in the last row
    par, _ = bench.grouped_oracle_leg(o, cfg, ops, bad)
    assert par["over"] == 1, par
    # past 10^11 multiply-adds (a stand-in config with a huge K): sampled
    cfg2, ops2 = _grouped(4, 160, 32, 16, 64)
    ref2, _, _ = o.grouped_gemm(ops2.a_codes, ops2.a_scales, ops2.b_codes, ops2.b_scales,
                                ops2.offsets, 1.0)
    big = types.SimpleNamespace(M=cfg2.M, N=cfg2.N, K=10 ** 10, alpha=1.0)
    par, stats = bench.grouped_oracle_leg(o, big, ops2, ref2)
    counts = np.diff(ops2.offsets)
    assert par["elements"].startswith("16 whole experts "), par["elements"]
    picked = ast.literal_eval(par["elements"][len("16 whole experts "):])
    nonempty = np.flatnonzero(counts)
    assert len(set(picked)) == 16 and all(counts[e] > 0 for e in picked)
    for e in (nonempty[0], nonempty[-1], int(np.argmax(counts))):
        assert int(e) in picked
    assert par["n"] == sum(int(counts[e]) for e in picked) * cfg2.N
    assert par["over"] == 0 and par["bit_exact_frac"] == 1.0


def test_roofline_binds_by_arithmetic_intensity_and_reports_the_other_resource():
    """Below the ridge (2.5 PF / 8 TB/s = 312.5 FLOP/B) the HBM roofline
    binds, above it the fp16 MFMA peak; the other resource's rate is beside
    it.  The decode projection (AI 3.5) and the saturation shape (AI 5,761)."""
    import bench
    for i, bound, other in ((2, "hbm", "mfma"), (5, "mfma", "hbm")):
        c = synth.config(i)
        r = bench.roofline_for(c, 1e-3)
        b, f = synth.algorithmic_bytes(c.M, c.N, c.K), synth.flops(c.M, c.N, c.K)
        assert r["bound"] == bound and r["other"]["resource"] == other
        gbps, tflops = b / 1e-3 / 1e9, f / 1e-3 / 1e12
        hbm = r if bound == "hbm" else r["other"]
        mfma = r if bound == "mfma" else r["other"]
        assert abs(hbm["achieved"] - gbps) < 1e-9 * gbps and hbm["unit"] == "GB/s"
        assert abs(mfma["achieved"] - tflops) < 1e-9 * tflops and mfma["unit"] == "TFLOP/s"
        assert abs(hbm["frac"] - gbps / 8000.0) < 1e-12 and abs(mfma["frac"] - tflops / 2500.0) < 1e-12
