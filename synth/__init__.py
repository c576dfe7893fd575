"""Seeded synthetic inputs for the NVFP4 block-scaled GEMM.

This module only MAKES inputs: it draws seeded fp32 matrices and quantises
them to NVFP4 (E2M1 codes packed two per byte, one E4M3 scale per 16-element
K-block), the format of "Peeling the Kernel Onion", section "The Benchmark
Design".  It holds none of the GEMM's arithmetic and is shared, as the only
common module, by the tests, the benchmark and the oracle's callers.

Workloads (M x N x K) stand in for the per-GPU GEMM shares of the model the
pages serve: hidden size 6144, MoE intermediate size 2048, eight-way tensor
parallel shares 768 and 256 ("Peeling the Kernel Onion", section "The
Benchmark Design"), about 16 tokens per expert at batch 512 (same page,
section "The Critical Connection to Real Inference"), batched shapes from
section "The Chain of Reasoning" and the largest shape of the size sweep.

Quantiser (per 16-element block of a row): scale = E4M3_RNE(amax / 6),
saturating at 448; amax == 0 gives scale 0 and zero codes; y = x / scale in
fp32; code = E2M1 round-to-nearest with ties to the even code, |y| > 6
saturates to +-6; the code keeps the sign of x.
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

# Non-negative finite FP8 E4M3 values, indexed by their byte (0x00..0x7E).
_E4M3_POS = np.array(
    [(f / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + f / 8.0) * 2.0 ** (e - 7)
     for e in range(16) for f in range(8)][:127], dtype=np.float64)
# Non-negative FP4 E2M1 magnitudes, indexed by the 3-bit magnitude code.
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def _nearest_even(table: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of an increasing table, ties to the even
    index; values beyond the last entry saturate to it."""
    mids = (table[1:] + table[:-1]) / 2.0
    idx = np.searchsorted(mids, v, side="left")
    tie = np.zeros(v.shape, dtype=bool)
    inside = idx < mids.shape[0]
    tie[inside] = v[inside] == mids[idx[inside]]
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return np.minimum(idx, table.shape[0] - 1)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Non-negative fp32/fp64 values -> E4M3 bytes (RNE, saturating at 448)."""
    v = np.asarray(x, dtype=np.float64)
    assert np.all(v >= 0)
    return _nearest_even(_E4M3_POS, v).astype(np.uint8)


def e4m3_value(byte: np.ndarray) -> np.ndarray:
    """Non-negative E4M3 bytes (0x00..0x7E) -> value (float64)."""
    return _E4M3_POS[np.asarray(byte, dtype=np.int64)]


def quantize_nvfp4(x: np.ndarray, workers: int | None = None):
    """fp32 [rows, K] -> (codes uint8 [rows, K/2], scales uint8 [rows, K/16]).
    Large inputs are processed in row chunks on a thread pool (the result
    does not depend on the chunking)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    assert K % 16 == 0
    chunk = max(1, (1 << 22) // K)
    if rows <= chunk:
        return _quantize_rows(x)
    from concurrent.futures import ThreadPoolExecutor
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)

    def work(r0):
        c, s = _quantize_rows(x[r0:r0 + chunk])
        codes[r0:r0 + chunk] = c
        scales[r0:r0 + chunk] = s

    n = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(work, range(0, rows, chunk)))
    return codes, scales


def _quantize_rows(x: np.ndarray):
    rows, K = x.shape
    blocks = x.reshape(rows, K // 16, 16)
    amax = np.max(np.abs(blocks), axis=2)
    scale_f32 = (amax / np.float32(6.0)).astype(np.float32)
    sbytes = e4m3_encode(scale_f32)
    sval = e4m3_value(sbytes).astype(np.float32)
    safe = np.where(sval > 0, sval, np.float32(1.0)).astype(np.float32)
    y = (blocks / safe[:, :, None]).astype(np.float32)
    y = np.where((sval > 0)[:, :, None], y, np.float32(0.0))
    mag = _nearest_even(_E2M1_POS, np.abs(y).astype(np.float64).ravel()).reshape(y.shape)
    sign = np.signbit(blocks).astype(np.uint8)
    codes = (mag.astype(np.uint8) | (sign << 3)).reshape(rows, K)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(sbytes)


@dataclass(frozen=True)
class GemmConfig:
    name: str
    M: int
    N: int
    K: int
    alpha: float
    sigma_b: float
    index: int          # 1-based workload number; seeds are 1000+i (A), 2000+i (B)
    description: str


CONFIGS = [
    GemmConfig("moe_up_tp8_b16", 16, 256, 6144, 1.0, 1.0, 1,
               "MoE up-projection eight-way share at 16 tokens per expert"),
    GemmConfig("decode_attn_proj", 1, 768, 6144, 0.5, 1.0, 2,
               "decode attention projection, eight-way share, batch 1"),
    GemmConfig("batched_attn_proj", 512, 768, 6144, 1.0, 1.0, 3,
               "batched attention projection, batch 512"),
    GemmConfig("moe_up_b512", 512, 2048, 6144, 1.0, 0.02, 4,
               "MoE up-projection at batch 512, weight-like B ~ N(0, 0.02)"),
    GemmConfig("saturation", 16384, 8192, 8192, 1.0, 1.0, 5,
               "compute-saturation shape"),
]


def config(i: int) -> GemmConfig:
    """Workload number i (1-based)."""
    return CONFIGS[i - 1]


@dataclass
class Operands:
    a_codes: np.ndarray
    a_scales: np.ndarray
    b_codes: np.ndarray
    b_scales: np.ndarray
    alpha: float
    M: int
    N: int
    K: int


def make_inputs(cfg: GemmConfig) -> Operands:
    """Seeded N(0,1) A (M x K) and N(0, sigma_b^2) B (N x K), quantised."""
    ga = np.random.Generator(np.random.PCG64(1000 + cfg.index))
    gb = np.random.Generator(np.random.PCG64(2000 + cfg.index))
    a = ga.standard_normal((cfg.M, cfg.K), dtype=np.float32)
    b = gb.standard_normal((cfg.N, cfg.K), dtype=np.float32)
    if cfg.sigma_b != 1.0:
        b = (b * np.float32(cfg.sigma_b)).astype(np.float32)
    ac, as_ = quantize_nvfp4(a)
    del a
    bc, bs = quantize_nvfp4(b)
    return Operands(ac, as_, bc, bs, cfg.alpha, cfg.M, cfg.N, cfg.K)


def random_operands(seed: int, M: int, N: int, K: int, alpha: float = 1.0,
                    scale_lo: int = 0x20, scale_hi: int = 0x48) -> Operands:
    """Uniformly random codes (all 16, incl. -0) and random scale bytes in
    [scale_lo, scale_hi] (positive, finite).  Used for parity at small shapes."""
    g = np.random.Generator(np.random.PCG64(seed))
    ac = g.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    bc = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    as_ = g.integers(scale_lo, scale_hi + 1, size=(M, K // 16), dtype=np.uint8)
    bs = g.integers(scale_lo, scale_hi + 1, size=(N, K // 16), dtype=np.uint8)
    return Operands(ac, as_, bc, bs, alpha, M, N, K)


def quantized_operands(seed: int, M: int, N: int, K: int, alpha: float = 1.0,
                       sigma_a: float = 1.0, sigma_b: float = 1.0) -> Operands:
    """Like make_inputs, for an arbitrary shape and seed."""
    g = np.random.Generator(np.random.PCG64(seed))
    a = (g.standard_normal((M, K), dtype=np.float32) * np.float32(sigma_a)).astype(np.float32)
    b = (g.standard_normal((N, K), dtype=np.float32) * np.float32(sigma_b)).astype(np.float32)
    ac, as_ = quantize_nvfp4(a)
    bc, bs = quantize_nvfp4(b)
    return Operands(ac, as_, bc, bs, alpha, M, N, K)


def operand_bytes(rows: int, K: int) -> int:
    """Unpadded size of one NVFP4 operand: a byte holds two 4-bit codes, and
    every 16-element block of a row carries one 1-byte scale."""
    codes = rows * K // 2
    scales = rows * (K // 16)
    return codes + scales


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """Bytes the GEMM must move at least once: both operands read and the
    bfloat16 output written (the traffic model of "Peeling the Kernel Onion",
    section "The Benchmark Design")."""
    return operand_bytes(M, K) + operand_bytes(N, K) + 2 * M * N


def flops(M: int, N: int, K: int) -> int:
    """Two operations (multiply, add) per term of the contraction."""
    return 2 * M * N * K


# ---------------------------------------------------------------------------
# Grouped (mixture-of-experts) workloads: every token is routed to top_k of
# the experts; the rows of A are the routed (token, expert) pairs in expert
# order and group g holds the rows of expert g.  The routing is a seeded
# uniform choice of top_k distinct experts per token (a stand-in for a
# router: no model or dataset is involved).  Sizes follow "Peeling the
# Kernel Onion", section "The Critical Connection to Real Inference" (256
# experts, 8 per token, 512 requests: about 16 tokens per expert) and the
# eight-way N share of the MoE up-projection of section "The Chain of
# Reasoning That Led to This Benchmark" (N = 2048 / 8, K = 6144).
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class GroupedConfig:
    name: str
    tokens: int
    experts: int
    top_k: int
    N: int
    K: int
    alpha: float
    index: int          # seeds: 1000+i (tokens), 2000+i (weights), 3000+i (routing)
    description: str

    @property
    def M(self) -> int:
        """Rows of A (routed token-expert pairs)."""
        return self.tokens * self.top_k


GROUPED_CONFIGS = [
    GroupedConfig("moe_up_grouped_e256", 512, 256, 8, 256, 6144, 1.0, 6,
                  "MoE up-projection eight-way share, all 256 experts in one launch, "
                  "512 tokens routed to 8 experts each (about 16 rows per expert)"),
    GroupedConfig("moe_up_grouped_e256_t4096", 4096, 256, 8, 256, 6144, 1.0, 7,
                  "the same layer for a prefill-sized batch: 4096 tokens routed to 8 of "
                  "256 experts each (about 128 rows per expert)"),
]


def grouped_config(name: str) -> GroupedConfig:
    for c in GROUPED_CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


@dataclass
class GroupedOperands:
    a_codes: np.ndarray    # [M, K/2]   rows in group order
    a_scales: np.ndarray   # [M, K/16]
    b_codes: np.ndarray    # [G, N, K/2]
    b_scales: np.ndarray   # [G, N, K/16]
    offsets: np.ndarray    # int32 [G + 1]: group g holds rows offsets[g] .. offsets[g+1]-1
    alpha: float
    M: int
    N: int
    K: int
    G: int


def moe_routing(seed: int, tokens: int, experts: int, top_k: int):
    """Seeded routing: each token picks top_k distinct experts uniformly.
    Returns (offsets int32 [experts + 1], token index of each routed row,
    rows sorted by expert then token)."""
    g = np.random.Generator(np.random.PCG64(seed))
    keys = g.random((tokens, experts))
    choice = np.argsort(keys, axis=1)[:, :top_k]             # [tokens, top_k]
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(tokens), top_k)
    order = np.lexsort((token, expert))
    counts = np.bincount(expert, minlength=experts)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return offsets, token[order]


def grouped_operands(seed: int, tokens: int, experts: int, top_k: int, N: int, K: int,
                     alpha: float = 1.0, offsets: np.ndarray | None = None,
                     token_of_row: np.ndarray | None = None) -> GroupedOperands:
    """Seeded N(0,1) token activations and expert weights, quantised; the
    quantised token rows are gathered into group order (quantisation is per
    row, so this equals quantising the gathered rows).  A routing may be
    passed in (offsets, token_of_row); else it is drawn with seed 3000+seed."""
    if offsets is None:
        offsets, token_of_row = moe_routing(3000 + seed, tokens, experts, top_k)
    ga = np.random.Generator(np.random.PCG64(1000 + seed))
    gb = np.random.Generator(np.random.PCG64(2000 + seed))
    x = ga.standard_normal((tokens, K), dtype=np.float32)
    tc, ts = quantize_nvfp4(x)
    del x
    a_codes = np.ascontiguousarray(tc[token_of_row])
    a_scales = np.ascontiguousarray(ts[token_of_row])
    b_codes = np.empty((experts, N, K // 2), np.uint8)
    b_scales = np.empty((experts, N, K // 16), np.uint8)
    for e in range(experts):
        w = gb.standard_normal((N, K), dtype=np.float32)
        b_codes[e], b_scales[e] = quantize_nvfp4(w)
    return GroupedOperands(a_codes, a_scales, b_codes, b_scales, np.asarray(offsets, np.int32),
                           alpha, int(offsets[-1]), N, K, experts)


def make_grouped_inputs(cfg: GroupedConfig) -> GroupedOperands:
    return grouped_operands(cfg.index, cfg.tokens, cfg.experts, cfg.top_k, cfg.N, cfg.K, cfg.alpha)


def grouped_algorithmic_bytes(M: int, N: int, K: int, G: int) -> int:
    """A (M rows) and the G weight operands (N rows each) read once, the
    bfloat16 output written once."""
    return operand_bytes(M, K) + G * operand_bytes(N, K) + 2 * M * N
