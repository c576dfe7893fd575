"""Host-side checks of the allocation-free entry point (no GPU needed): the
scratch a plan needs, and the refusal of a shape whose plan needs more than
the static array holds, before any device call."""
import ctypes

import pytest

import block_scaled_fp4_04_amd as nv


def test_scratch_bytes_follow_the_plan():
    # no split-K: nothing needed
    assert nv.noalloc_scratch_bytes(1, 768, 6144) == (0, True)
    # a split-K plan: its counters and FP32 partial tiles
    need, fits = nv.noalloc_scratch_bytes(64, 200, 16384)
    p = nv.plan(64, 200, 16384)
    assert p["split_k"] > 1 and fits and need > 0
    # a tail round of 6144^3: more partial tiles than the array holds
    need, fits = nv.noalloc_scratch_bytes(6144, 6144, 6144)
    assert not fits and need > nv.NOALLOC_SCRATCH_BYTES
    with pytest.raises(nv.Nvfp4Error):
        nv.noalloc_scratch_bytes(1, 768, 100)   # K % 16 != 0


def test_refused_before_any_device_call():
    L = nv.lib()
    p = 0x100000   # aligned stand-in addresses: the call must return before using them
    assert L.nvfp4_gemm_noalloc(p, p, p, p, 1.0, p, 6144, 6144, 6144, None) == nv.ERR_SCRATCH
    assert L.nvfp4_gemm_noalloc(p, p, p, p, 1.0, p, 16, 256, 100, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_gemm_noalloc(None, p, p, p, 1.0, p, 16, 256, 6144, None) == nv.ERR_INVALID_VALUE
    assert L.nvfp4_gemm_noalloc(p + 8, p, p, p, 1.0, p, 16, 256, 6144, None) == nv.ERR_MISALIGNED
    assert L.nvfp4_noalloc_scratch_bytes(16, 256, 6144, None) == nv.ERR_INVALID_VALUE
    b = ctypes.c_size_t()
    assert L.nvfp4_noalloc_scratch_bytes(0, 256, 6144, ctypes.byref(b)) == nv.ERR_INVALID_VALUE
    assert "scratch" in nv.status_string(nv.ERR_SCRATCH)
