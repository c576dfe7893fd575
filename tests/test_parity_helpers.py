"""CPU checks of the parity helpers used for outputs too large to check
whole (oracle/parity.py): the element sets and the sampled comparison."""
import numpy as np

import synth
from oracle import oracle as orc
from parity import check_sample, large_sample, tile_origin


def test_tile_order_covers_every_tile_once():
    for tm, tn in ((64, 32), (3, 5), (9, 2), (8, 8)):
        seen = {tile_origin(t, tm, tn) for t in range(tm * tn)}
        assert seen == {(m * 256, n * 256) for m in range(tm) for n in range(tn)}


def test_large_sample_of_the_saturation_shape():
    s = large_sample(16384, 8192)
    assert s["rows"] == [0, 255, 256, 16383] and s["cols"] == [0, 255, 256, 8191]
    # 2048 tiles, 256 per XCD: each XCD's range starts on a new group of 8 tile rows
    assert s["tiles"] == [(2048 * x, 0) for x in range(8)] + [(16128, 7936)]
    assert len(s["points"][0]) == 4096


def test_check_sample_finds_a_wrong_element_it_covers():
    o = orc.load()
    ops = synth.random_operands(11, 600, 520, 64, alpha=0.5)
    bits, _, _ = o.gemm(ops.a_codes, ops.a_scales, ops.b_codes, ops.b_scales, ops.alpha)
    s = large_sample(600, 520, random_points=64)
    assert s["tiles"] == [(0, 0), (512, 512)]   # 9 tiles: no XCD ranges, first and last
    r = check_sample(o, ops, bits.copy(), s)
    assert r["over"] == 0 and r["bit_exact_frac"] == 1.0
    assert r["n"] == 4 * 520 + 4 * 600 + 256 * 256 + 88 * 8 + 64
    for m, n in ((255, 17), (300, 519), (10, 10), (550, 515)):   # a row, a column, two tiles
        bad = bits.copy()
        bad[m, n] ^= 0x0100
        assert check_sample(o, ops, bad, s)["over"] >= 1, (m, n)
