"""Element-by-element comparison of GPU results with the CPU oracle."""
from __future__ import annotations

import numpy as np

from oracle import oracle as orc


def compare(gpu_bits: np.ndarray, oracle_bits: np.ndarray, exact: np.ndarray, mag: np.ndarray,
            alpha: float) -> dict:
    """Per-element bound |gpu - oracle| <= ulp_bf16(oracle) + 1e-5*|alpha|*sum|a'b'|,
    where ulp is taken at the larger of the exact and the rounded oracle value
    (so a result on either side of a power of two gets the wider spacing).
    Returns counts; 'over' must be 0."""
    g = orc.bf16_bits_to_float(np.asarray(gpu_bits, np.uint16).astype(np.uint32) & 0xFFFF)
    o = orc.bf16_bits_to_float(np.asarray(oracle_bits, np.uint16))
    ref = np.maximum(np.abs(exact), np.abs(o))
    tol = orc.bf16_ulp(ref) + 1e-5 * abs(alpha) * mag
    err = np.abs(g - o)
    nan_mismatch = int(np.sum(np.isnan(g) != np.isnan(o)))
    finite = ~np.isnan(g) & ~np.isnan(o)
    over = int(np.sum(err[finite] > tol[finite])) + nan_mismatch
    same = (np.asarray(gpu_bits, np.uint16) == np.asarray(oracle_bits, np.uint16)) | (
        (g == 0) & (o == 0))
    ratio = float(np.max(err[finite] / tol[finite])) if np.any(finite) else 0.0
    return {"n": int(g.size), "over": over, "bit_exact": int(np.sum(same)),
            "bit_exact_frac": float(np.mean(same)) if g.size else 1.0,
            "max_err_over_tol": ratio, "all_zero": bool(np.all(g == 0))}
