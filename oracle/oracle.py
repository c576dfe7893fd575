"""Python handle on the plain-C oracle (nvfp4_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module; the product path never does.  The
oracle shares no code with the HIP library.

The oracle computes C = alpha * (A . B^T) for NVFP4 operands in their
canonical layout (codes [rows][K/2], element 2j in the low nibble of byte j;
scales [rows][K/16]), accumulating in fp64 and rounding once to bfloat16.
The format facts follow "Peeling the Kernel Onion", section "The Benchmark
Design" (uint8 holding two codes, one FP8 scale per 16 elements, 2-byte
output) and "The SM120 FP4 Kernel Disaster", section "Input Knowledge
Required", item 3.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(out_path: str = LIB_PATH, mutant: int = 0, extra_flags: tuple[str, ...] = ()) -> str:
    """Compile the oracle with gcc (OpenMP, -O2).  ``mutant`` != 0 plants one
    deliberate mistake (see the ORACLE_MUTANT cases in the C source);
    ``extra_flags`` go to gcc as given (for instance sanitizers)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", *extra_flags, _SRC, "-o",
           out_path, "-lm"]
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    tmp = out_path + f".tmp{os.getpid()}"
    cmd[cmd.index(out_path)] = tmp
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build_mutant(mutant: int, directory: str | None = None) -> str:
    d = directory or tempfile.mkdtemp(prefix="oracle_mutant_")
    return build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant)


def _setup(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_e2m1.restype = ctypes.c_double
    lib.oracle_e2m1.argtypes = [ctypes.c_uint]
    lib.oracle_e4m3.restype = ctypes.c_double
    lib.oracle_e4m3.argtypes = [ctypes.c_uint]
    lib.oracle_bf16.restype = ctypes.c_uint16
    lib.oracle_bf16.argtypes = [ctypes.c_double]
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_mutant_id.restype = ctypes.c_int
    lib.oracle_element.restype = ctypes.c_double
    lib.oracle_element.argtypes = [_u8p, _u8p, _i64, _i64, _i64]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_float, _i64, _i64, _i64,
                                _u16p, _f64p, _f64p]
    lib.oracle_quantize.restype = ctypes.c_int
    lib.oracle_quantize.argtypes = [ctypes.POINTER(ctypes.c_float), _i64, _i64, _i64, _u8p, _u8p]
    lib.oracle_gemm_points.restype = ctypes.c_int
    lib.oracle_gemm_points.argtypes = [_u8p, _u8p, _u8p, _u8p, ctypes.c_float, _i64, _i64, _i64,
                                       _i64p, _i64p, _i64, _u16p, _f64p, _f64p]
    return lib


_LIB: ctypes.CDLL | None = None


def load(path: str | None = None) -> "Oracle":
    """Load the oracle library (building it first if it is not there)."""
    global _LIB
    if path is not None:
        return Oracle(_setup(ctypes.CDLL(path)))
    if _LIB is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _LIB = _setup(ctypes.CDLL(LIB_PATH))
    return Oracle(_LIB)


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


class Oracle:
    """Thin wrapper; every method takes canonical numpy uint8 arrays."""

    def __init__(self, lib: ctypes.CDLL):
        self.lib = lib

    @property
    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    @property
    def mutant(self) -> int:
        return int(self.lib.oracle_mutant_id())

    def e2m1(self, code: int) -> float:
        return float(self.lib.oracle_e2m1(code))

    def e4m3(self, byte: int) -> float:
        return float(self.lib.oracle_e4m3(byte))

    def element(self, codes: np.ndarray, scales: np.ndarray, r: int, k: int) -> float:
        K = 2 * codes.shape[1]
        return float(self.lib.oracle_element(_ptr(codes, _u8p), _ptr(scales, _u8p), K, r, k))

    def bf16(self, x: float) -> int:
        return int(self.lib.oracle_bf16(float(x)))

    @staticmethod
    def _check(a_codes, a_scales, b_codes, b_scales):
        M, kh = a_codes.shape
        N = b_codes.shape[0]
        K = 2 * kh
        for arr in (a_codes, a_scales, b_codes, b_scales):
            assert arr.dtype == np.uint8 and arr.flags.c_contiguous
        assert b_codes.shape == (N, K // 2), "A and B must share K"
        assert a_scales.shape == (M, K // 16) and b_scales.shape == (N, K // 16)
        return M, N, K

    def gemm(self, a_codes, a_scales, b_codes, b_scales, alpha: float = 1.0, want_exact=True):
        """Returns (bf16 bits uint16 [M,N], alpha*S fp64 [M,N], T fp64 [M,N])."""
        M, N, K = self._check(a_codes, a_scales, b_codes, b_scales)
        out = np.zeros((M, N), np.uint16)
        exact = np.zeros((M, N), np.float64) if want_exact else None
        mag = np.zeros((M, N), np.float64) if want_exact else None
        rc = self.lib.oracle_gemm(_ptr(a_codes, _u8p), _ptr(a_scales, _u8p), _ptr(b_codes, _u8p),
                                  _ptr(b_scales, _u8p), ctypes.c_float(alpha), M, N, K,
                                  _ptr(out, _u16p),
                                  _ptr(exact, _f64p) if want_exact else None,
                                  _ptr(mag, _f64p) if want_exact else None)
        if rc != 0:
            raise ValueError(f"oracle_gemm failed with {rc}")
        return out, exact, mag

    def gemm_points(self, a_codes, a_scales, b_codes, b_scales, alpha, ms, ns):
        """Selected elements (ms[p], ns[p]); returns (bits, alpha*S, T) as 1-D arrays."""
        M, N, K = self._check(a_codes, a_scales, b_codes, b_scales)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        P = ms.shape[0]
        out = np.zeros(P, np.uint16)
        exact = np.zeros(P, np.float64)
        mag = np.zeros(P, np.float64)
        rc = self.lib.oracle_gemm_points(_ptr(a_codes, _u8p), _ptr(a_scales, _u8p),
                                         _ptr(b_codes, _u8p), _ptr(b_scales, _u8p),
                                         ctypes.c_float(alpha), M, N, K, _ptr(ms, _i64p),
                                         _ptr(ns, _i64p), P, _ptr(out, _u16p),
                                         _ptr(exact, _f64p), _ptr(mag, _f64p))
        if rc != 0:
            raise ValueError(f"oracle_gemm_points failed with {rc}")
        return out, exact, mag


    def quantize(self, x: np.ndarray):
        """fp32 [rows, K] -> (codes uint8 [rows, K/2], scales uint8 [rows, K/16]):
        per 16-element block, scale = E4M3 nearest-even of fp32(amax / 6)
        (saturating at 448), code = E2M1 nearest-even of fp32(x / scale) with
        the sign of x (see oracle_quantize in the C source)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        rows, K = x.shape
        codes = np.zeros((rows, K // 2), np.uint8)
        scales = np.zeros((rows, K // 16), np.uint8)
        rc = self.lib.oracle_quantize(x.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), rows, K, K,
                                      _ptr(codes, _u8p), _ptr(scales, _u8p))
        if rc != 0:
            raise ValueError(f"oracle_quantize failed with {rc}")
        return codes, scales

    def grouped_gemm(self, a_codes, a_scales, b_codes, b_scales, offsets, alpha: float = 1.0):
        """Grouped GEMM (mixture-of-experts layer) by its definition: group g
        owns rows offsets[g] .. offsets[g+1]-1 of A and of C, and those rows
        are the ordinary GEMM of the group's A rows with the group's own
        weight operand B_g = b_codes[g], b_scales[g] ("Peeling the Kernel
        Onion", section "The Critical Connection to Real Inference": each
        expert multiplies the tokens routed to it).  b_codes is [G, N, K/2],
        b_scales [G, N, K/16]; offsets has G + 1 non-decreasing entries from 0
        to the number of rows of A.  Returns (bits, alpha*S, T) for all rows."""
        offsets = np.asarray(offsets, dtype=np.int64)
        G = b_codes.shape[0]
        M, N = a_codes.shape[0], b_codes.shape[1]
        assert offsets.shape == (G + 1,) and offsets[0] == 0 and offsets[-1] == M
        assert np.all(np.diff(offsets) >= 0)
        bits = np.zeros((M, N), np.uint16)
        exact = np.zeros((M, N), np.float64)
        mag = np.zeros((M, N), np.float64)
        for g in range(G):
            r0, r1 = int(offsets[g]), int(offsets[g + 1])
            if r0 == r1:
                continue
            gb, ge, gm = self.gemm(np.ascontiguousarray(a_codes[r0:r1]),
                                   np.ascontiguousarray(a_scales[r0:r1]),
                                   np.ascontiguousarray(b_codes[g]),
                                   np.ascontiguousarray(b_scales[g]), alpha)
            bits[r0:r1], exact[r0:r1], mag[r0:r1] = gb, ge, gm
        return bits, exact, mag


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    u32 = np.asarray(bits, dtype=np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 values at x: 2^(max(floor(log2|x|), -126) - 7); at 0 it is 2^-133."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.where(ax > 0, np.floor(np.log2(np.where(ax > 0, ax, 1.0))), -126.0)
    e = np.maximum(e, -126.0)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def tolerance(exact: np.ndarray, mag: np.ndarray, alpha: float) -> np.ndarray:
    """Per-element parity bound: one bf16 ulp of the oracle value plus
    1e-5 * |alpha| * sum_k |a'_k b'_k|."""
    return bf16_ulp(exact) + 1e-5 * abs(alpha) * mag
