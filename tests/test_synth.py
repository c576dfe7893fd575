"""The input quantiser against a library routine and its stated rules."""
import numpy as np
import torch

import synth


def test_e4m3_encode_matches_torch_rne():
    g = np.random.default_rng(0)
    v = np.abs(g.standard_normal(20000)).astype(np.float32) * np.float32(2.0) ** g.integers(
        -14, 9, 20000).astype(np.float32)
    v = v[v <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.e4m3_encode(v), ref)
    mids = ((synth._E4M3_POS[1:] + synth._E4M3_POS[:-1]) / 2).astype(np.float32)
    ref = torch.from_numpy(mids).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(synth.e4m3_encode(mids), ref)
    assert synth.e4m3_encode(np.array([1000.0]))[0] == 0x7E   # saturates at 448


def test_e2m1_ties_to_even_and_saturation():
    # one block: amax 6 -> scale 1.0, so y = x
    x = np.array([[6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.1, -6.0,
                   2.9, 0.0, -0.0, 4.1]], np.float32)
    codes, scales = synth.quantize_nvfp4(x)
    assert scales[0, 0] == 0x38
    c = np.empty(16, np.uint8)
    c[0::2], c[1::2] = codes[0] & 0xF, codes[0] >> 4
    want = [7, 0, 2, 2, 4, 4, 6, 6, 8, 14, 0, 15, 5, 0, 8, 6]
    assert c.tolist() == want


def test_zero_block_and_saturating_scale_rounding():
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = 7.0                    # amax 7 -> 7/6 -> E4M3 1.125 (0x39); 7/1.125 > 6 -> code 7
    codes, scales = synth.quantize_nvfp4(x)
    assert scales[0, 0] == 0 and not codes[0, :8].any()
    assert scales[0, 1] == 0x39
    assert np.all(codes[0, 8:] == 0x77)


def test_config_value_structure():
    ops = synth.make_inputs(synth.config(4))
    sub = np.mean((ops.b_scales >> 3) == 0)
    assert sub > 0.99                  # B ~ N(0, 0.02): almost all scales subnormal
    ops1 = synth.make_inputs(synth.config(1))
    assert ops1.a_codes.shape == (16, 3072) and ops1.b_scales.shape == (256, 384)
