"""Python binding of the gfx950 NVFP4 block-scaled GEMM library (libnvfp4.so).

Argument marshalling only: every step of the GEMM runs in the HIP kernels
behind the C ABI of ``include/nvfp4.h``; PyTorch supplies device memory and
the current stream.  There is no fallback: if the library is missing, every
call raises.

On first use the library is given the tuned plan table shipped beside it
(``plan_table_gfx950.json``, written by ``python -m
block_scaled_fp4_04_amd.tune``); the environment variable NVFP4_PLAN_TABLE
names another table file, or ``off`` for the library's own rules only.

    C = alpha * (A . B^T)
A is M x K and B is N x K, both E2M1 codes packed two per byte with one
E4M3 scale per 16 elements, alpha is FP32 and C is bfloat16 M x N ("Peeling
the Kernel Onion", sections "The Benchmark Design" and "The Chain of
Reasoning").
"""
from __future__ import annotations

import ctypes
import os
import warnings
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnvfp4.so")
PLAN_TABLE_PATH = os.path.join(_PKG, "plan_table_gfx950.json")

OK = 0
ERR_INVALID_VALUE = 1
ERR_MISALIGNED = 2
ERR_UNSUPPORTED = 3
ERR_HIP = 4
ERR_ALLOC = 5
ERR_CAPTURE = 6
ERR_STATE = 7
ERR_DEVICE_FLAGS = 8
ERR_SCRATCH = 9

FLAG_HANDOFF = 1
NOALLOC_SCRATCH_BYTES = 32 << 20
NOALLOC_MAX_COUNTERS = 16384

PATH_AUTO = 0
PATH_TILE = 1
PATH_SKINNY = 2
PATH_WSPLIT = 3
PATH_GEMV = 4
INPUT_F32 = 0     # element types of nvfp4_gemm_quantized's activation rows
INPUT_BF16 = 1
PATH_NAMES = {PATH_TILE: "tile", PATH_SKINNY: "skinny", PATH_WSPLIT: "wsplit", PATH_GEMV: "gemv"}

PLAN_HEURISTIC = 0
PLAN_TABLE = 1

EXPORTS = ["nvfp4_status_string", "nvfp4_version", "nvfp4_packed_size", "nvfp4_pack",
           "nvfp4_unpack", "nvfp4_init", "nvfp4_shutdown", "nvfp4_gemm",
           "nvfp4_gemm_with_plan", "nvfp4_plan", "nvfp4_plan_table_load",
           "nvfp4_plan_table_clear", "nvfp4_build_id", "nvfp4_grouped_gemm",
           "nvfp4_grouped_gemm_with_plan", "nvfp4_quantize",
           "nvfp4_sequence_create", "nvfp4_sequence_add_gemm", "nvfp4_sequence_add_grouped_gemm",
           "nvfp4_sequence_add_quantize", "nvfp4_sequence_finalize", "nvfp4_sequence_launch",
           "nvfp4_quantize_bf16", "nvfp4_sequence_add_quantize_bf16", "nvfp4_gemm_quantized",
           "nvfp4_sequence_add_gemm_quantized",
           "nvfp4_sequence_destroy", "nvfp4_probe_empty", "nvfp4_probe_chase",
           "nvfp4_probe_mfma", "nvfp4_probe_read", "nvfp4_device_flags",
           "nvfp4_debug_set_handoff_polls", "nvfp4_gemm_noalloc", "nvfp4_noalloc_scratch_bytes"]


class _PlanT(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("tail_tiles", ctypes.c_int32),
                ("tail_split", ctypes.c_int32), ("source", ctypes.c_int32)]


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


_u8p = ctypes.POINTER(ctypes.c_uint8)
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_lib: ctypes.CDLL | None = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m block_scaled_fp4_04_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_status_string.argtypes = [ctypes.c_int]
        L.nvfp4_version.restype = ctypes.c_int
        L.nvfp4_packed_size.restype = ctypes.c_int
        L.nvfp4_packed_size.argtypes = [_i64, _i64, ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.POINTER(ctypes.c_size_t)]
        L.nvfp4_pack.restype = ctypes.c_int
        L.nvfp4_pack.argtypes = [_u8p, _u8p, _i64, _i64, _u8p, _u8p]
        L.nvfp4_unpack.restype = ctypes.c_int
        L.nvfp4_unpack.argtypes = [_u8p, _u8p, _i64, _i64, _u8p, _u8p]
        L.nvfp4_init.restype = ctypes.c_int
        L.nvfp4_init.argtypes = [ctypes.c_int]
        L.nvfp4_shutdown.restype = None
        L.nvfp4_gemm.restype = ctypes.c_int
        L.nvfp4_gemm.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64, _i64, _vp]
        L.nvfp4_gemm_with_plan.restype = ctypes.c_int
        L.nvfp4_gemm_with_plan.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64,
                                           _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]
        for f in ("nvfp4_quantize", "nvfp4_quantize_bf16"):
            getattr(L, f).restype = ctypes.c_int
            getattr(L, f).argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp]
        L.nvfp4_probe_empty.restype = ctypes.c_int
        L.nvfp4_probe_empty.argtypes = [_i64, _i64, _vp]
        L.nvfp4_probe_chase.restype = ctypes.c_int
        L.nvfp4_probe_chase.argtypes = [_vp, _i64, _i64, _vp, _vp]
        L.nvfp4_probe_mfma.restype = ctypes.c_int
        L.nvfp4_probe_mfma.argtypes = [_i64, _i64, _vp, _vp]
        L.nvfp4_probe_read.restype = ctypes.c_int
        L.nvfp4_probe_read.argtypes = [_vp, _i64, _i64, _vp, _vp]
        L.nvfp4_device_flags.restype = ctypes.c_int
        L.nvfp4_device_flags.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
        L.nvfp4_debug_set_handoff_polls.restype = ctypes.c_int
        L.nvfp4_debug_set_handoff_polls.argtypes = [ctypes.c_uint32]
        L.nvfp4_gemm_noalloc.restype = ctypes.c_int
        L.nvfp4_gemm_noalloc.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64,
                                         _i64, _vp]
        L.nvfp4_noalloc_scratch_bytes.restype = ctypes.c_int
        L.nvfp4_noalloc_scratch_bytes.argtypes = [_i64, _i64, _i64,
                                                  ctypes.POINTER(ctypes.c_size_t)]
        L.nvfp4_grouped_gemm.restype = ctypes.c_int
        L.nvfp4_grouped_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, ctypes.c_float, _vp, _i64,
                                         _i64, _i64, _vp]
        L.nvfp4_grouped_gemm_with_plan.restype = ctypes.c_int
        L.nvfp4_grouped_gemm_with_plan.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, ctypes.c_float,
                                                   _vp, _i64, _i64, _i64, ctypes.c_int, _vp]
        L.nvfp4_gemm_quantized.restype = ctypes.c_int
        L.nvfp4_gemm_quantized.argtypes = [_vp, ctypes.c_int, _i64, _vp, _vp, ctypes.c_float, _vp,
                                           _i64, _i64, _i64, _vp]
        L.nvfp4_sequence_add_gemm_quantized.restype = ctypes.c_int
        L.nvfp4_sequence_add_gemm_quantized.argtypes = [_vp, _vp, ctypes.c_int, _i64, _vp, _vp,
                                                        ctypes.c_float, _vp, _i64, _i64, _i64]
        L.nvfp4_plan.restype = ctypes.c_int
        L.nvfp4_plan.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_PlanT)]
        L.nvfp4_plan_table_load.restype = ctypes.c_int
        L.nvfp4_plan_table_load.argtypes = [ctypes.c_char_p, ctypes.POINTER(_i64),
                                            ctypes.POINTER(ctypes.c_int)]
        L.nvfp4_plan_table_clear.restype = None
        L.nvfp4_build_id.restype = ctypes.c_char_p
        L.nvfp4_sequence_create.restype = ctypes.c_int
        L.nvfp4_sequence_create.argtypes = [ctypes.POINTER(_vp)]
        L.nvfp4_sequence_add_gemm.restype = ctypes.c_int
        L.nvfp4_sequence_add_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _i64,
                                              _i64, _i64]
        L.nvfp4_sequence_add_grouped_gemm.restype = ctypes.c_int
        L.nvfp4_sequence_add_grouped_gemm.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                                      ctypes.c_float, _vp, _i64, _i64, _i64]
        for f in ("nvfp4_sequence_add_quantize", "nvfp4_sequence_add_quantize_bf16"):
            getattr(L, f).restype = ctypes.c_int
            getattr(L, f).argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _vp]
        for f in ("nvfp4_sequence_finalize", "nvfp4_sequence_destroy"):
            getattr(L, f).restype = ctypes.c_int
            getattr(L, f).argtypes = [_vp]
        L.nvfp4_sequence_launch.restype = ctypes.c_int
        L.nvfp4_sequence_launch.argtypes = [_vp, _vp]
        _lib = L
        load_default_plan_table()
    return _lib


def load_default_plan_table() -> int:
    """Give the library the table named by NVFP4_PLAN_TABLE, else the one
    shipped beside it (if present); ``off`` loads none.  Returns the number
    of entries loaded."""
    table = os.environ.get("NVFP4_PLAN_TABLE", "")
    if table.lower() == "off":
        return 0
    path = table or PLAN_TABLE_PATH
    if not table and not os.path.exists(path):
        return 0
    return load_plan_table(path)[0]


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(int(status)).decode()


def version() -> int:
    return int(lib().nvfp4_version())


def packed_size(rows: int, K: int) -> tuple[int, int]:
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    st = lib().nvfp4_packed_size(rows, K, ctypes.byref(cb), ctypes.byref(sb))
    if st:
        raise Nvfp4Error(st, f"nvfp4_packed_size(rows={rows}, K={K})")
    return cb.value, sb.value


def _check_canonical(codes: np.ndarray, scales: np.ndarray) -> tuple[int, int]:
    if codes.dtype != np.uint8 or scales.dtype != np.uint8 or codes.ndim != 2 or scales.ndim != 2:
        raise ValueError("codes and scales must be 2-D uint8 arrays")
    rows, kh = codes.shape
    K = 2 * kh
    if scales.shape != (rows, K // 16) or K % 16:
        raise ValueError(f"scales shape {scales.shape} does not match codes {codes.shape} "
                         "(one scale per 16 elements, K % 16 == 0)")
    return rows, K


def pack(codes: np.ndarray, scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Canonical host arrays -> packed host arrays (nvfp4_pack)."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    rows, K = _check_canonical(codes, scales)
    cb, sb = packed_size(rows, K)
    pc = np.empty(cb, np.uint8)
    ps = np.empty(sb, np.uint8)
    st = lib().nvfp4_pack(codes.ctypes.data_as(_u8p), scales.ctypes.data_as(_u8p), rows, K,
                          pc.ctypes.data_as(_u8p), ps.ctypes.data_as(_u8p))
    if st:
        raise Nvfp4Error(st, "nvfp4_pack")
    return pc, ps


def unpack(packed_codes: np.ndarray, packed_scales: np.ndarray, rows: int, K: int):
    """Packed host arrays -> canonical (codes [rows, K/2], scales [rows, K/16])."""
    packed_codes = np.ascontiguousarray(packed_codes, dtype=np.uint8)
    packed_scales = np.ascontiguousarray(packed_scales, dtype=np.uint8)
    cb, sb = packed_size(rows, K)
    if packed_codes.size != cb or packed_scales.size != sb:
        raise ValueError("packed buffers have the wrong size")
    codes = np.empty((rows, K // 2), np.uint8)
    scales = np.empty((rows, K // 16), np.uint8)
    st = lib().nvfp4_unpack(packed_codes.ctypes.data_as(_u8p), packed_scales.ctypes.data_as(_u8p),
                            rows, K, codes.ctypes.data_as(_u8p), scales.ctypes.data_as(_u8p))
    if st:
        raise Nvfp4Error(st, "nvfp4_unpack")
    return codes, scales


def tile_code(path: int, tile_m: int, tile_n: int) -> int:
    """The ``tile`` argument of nvfp4_gemm_with_plan that names a path's
    tile: the edge for PATH_TILE, rows x columns / 64 for PATH_WSPLIT
    (16, 32, 64, 128 for 32 x 32, 64 x 32, 64 x 64, 128 x 64), else 0."""
    if path == PATH_TILE:
        return tile_m
    if path == PATH_WSPLIT:
        return tile_m * tile_n // 64
    return 0


def plan(M: int, N: int, K: int) -> dict:
    """The plan nvfp4_gemm uses for the shape (path, tile, split-K, and
    whether it came from the tuned table); ``tile`` is its tile as
    nvfp4_gemm_with_plan takes it."""
    p = _PlanT()
    st = lib().nvfp4_plan(M, N, K, ctypes.byref(p))
    if st:
        raise Nvfp4Error(st, "nvfp4_plan")
    return {"path": p.path, "split_k": p.split_k, "tile_m": p.tile_m, "tile_n": p.tile_n,
            "tile": tile_code(p.path, p.tile_m, p.tile_n),
            "tail_tiles": p.tail_tiles, "tail_split": p.tail_split, "source": p.source}


def build_id() -> str:
    return lib().nvfp4_build_id().decode()


def load_plan_table(path: str) -> tuple[int, bool]:
    """Load a tuned plan table (JSON) into the library; returns (entries,
    same_build).  Warns when the table was timed on other kernels."""
    n, same = _i64(), ctypes.c_int()
    st = lib().nvfp4_plan_table_load(os.fsencode(path), ctypes.byref(n), ctypes.byref(same))
    if st:
        raise Nvfp4Error(st, f"nvfp4_plan_table_load({path})")
    if not same.value:
        warnings.warn(f"plan table {path} was timed on other kernels than build "
                      f"{build_id()}; its choices are valid but may not be the fastest",
                      stacklevel=2)
    return n.value, bool(same.value)


def clear_plan_table() -> None:
    lib().nvfp4_plan_table_clear()


def init(device: int = 0) -> None:
    st = lib().nvfp4_init(device)
    if st:
        raise Nvfp4Error(st, f"nvfp4_init({device})")


def shutdown() -> None:
    lib().nvfp4_shutdown()


@dataclass
class PackedOperand:
    """One GEMM operand in the packed layout, resident on a device.
    ``codes``/``scales`` are uint8 torch tensors; ``rows`` x ``K`` is the
    logical shape."""
    codes: "object"
    scales: "object"
    rows: int
    K: int

    def check(self, name: str) -> None:
        import torch
        need_c, need_s = packed_size(self.rows, self.K)
        for what, t, need in ((".codes", self.codes, need_c), (".scales", self.scales, need_s)):
            if t.dtype != torch.uint8 or t.numel() != need or not t.is_contiguous():
                raise ValueError(f"{name}{what} must be a contiguous uint8 tensor of {need} bytes")


def to_device(codes: np.ndarray, scales: np.ndarray, device="cuda") -> PackedOperand:
    """Pack canonical host arrays and copy them to ``device``."""
    import torch
    rows, K = _check_canonical(codes, scales)
    pc, ps = pack(codes, scales)
    return PackedOperand(torch.from_numpy(pc).to(device), torch.from_numpy(ps).to(device), rows, K)


def _stream_handle(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def gemm(a: PackedOperand, b: PackedOperand, alpha: float = 1.0, out=None,
         path: int = PATH_AUTO, split_k: int = 0, stream=None, tile: int = 0):
    """C = alpha * (A . B^T) as an M x N bfloat16 tensor on A's device.
    ``path``, ``tile`` and ``split_k`` force a launch plan as
    nvfp4_gemm_with_plan does (0 = the library's choice).  Raises ValueError
    when A and B do not share K (a mismatch is an error, not a silent
    result)."""
    import torch
    if a.K != b.K:
        raise ValueError(f"K dimension mismatch: A has K={a.K}, B has K={b.K}")
    M, N, K = a.rows, b.rows, a.K
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape ({M}, {N})")
    a.check("a")
    b.check("b")
    st = lib().nvfp4_gemm_with_plan(a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
                                    b.scales.data_ptr(), float(alpha), out.data_ptr(), M, N, K,
                                    int(path), int(tile), int(split_k), _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_gemm(M={M}, N={N}, K={K})")
    return out


def gemm_noalloc(a: PackedOperand, b: PackedOperand, alpha: float = 1.0, out=None, stream=None):
    """C = alpha * (A . B^T) through nvfp4_gemm_noalloc: the plan and result
    of gemm(), with the split-K workspace in the library's static device
    array instead of an allocation (``out`` given: nothing is allocated by
    this call).  Raises Nvfp4Error (status ERR_SCRATCH) for a shape whose
    plan needs more scratch than the array holds."""
    import torch
    if a.K != b.K:
        raise ValueError(f"K dimension mismatch: A has K={a.K}, B has K={b.K}")
    M, N, K = a.rows, b.rows, a.K
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape ({M}, {N})")
    a.check("a")
    b.check("b")
    st = lib().nvfp4_gemm_noalloc(a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
                                  b.scales.data_ptr(), float(alpha), out.data_ptr(), M, N, K,
                                  _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_gemm_noalloc(M={M}, N={N}, K={K})")
    return out


def noalloc_scratch_bytes(M: int, N: int, K: int) -> tuple[int, bool]:
    """(scratch bytes the shape's plan needs, whether nvfp4_gemm_noalloc
    accepts it)."""
    b = ctypes.c_size_t()
    st = lib().nvfp4_noalloc_scratch_bytes(M, N, K, ctypes.byref(b))
    if st not in (OK, ERR_SCRATCH):
        raise Nvfp4Error(st, f"nvfp4_noalloc_scratch_bytes(M={M}, N={N}, K={K})")
    return b.value, st == OK


def device_flags() -> int:
    """Synchronise the current device and return (and clear) the error
    flags its kernels raised (FLAG_* bits; 0 = none)."""
    f = ctypes.c_uint32()
    st = lib().nvfp4_device_flags(ctypes.byref(f))
    if st not in (OK, ERR_DEVICE_FLAGS):
        raise Nvfp4Error(st, "nvfp4_device_flags")
    return int(f.value)


def set_handoff_polls(polls: int | None) -> None:
    """Test hook: poll budget of a two-way split-K hand-off for calls
    planned from now on (None restores the default)."""
    lib().nvfp4_debug_set_handoff_polls(0xFFFFFFFF if polls is None else int(polls))


def gemm_raw(a_codes: int, a_scales: int, b_codes: int, b_scales: int, alpha: float, out: int,
             M: int, N: int, K: int, stream: int | None = None) -> int:
    """Direct call of nvfp4_gemm with raw device addresses; returns the status."""
    return int(lib().nvfp4_gemm(a_codes, a_scales, b_codes, b_scales, float(alpha), out, M, N, K,
                                stream))


@dataclass
class PackedGroups:
    """The weight operands of a grouped GEMM, each ``rows`` x ``K``, packed
    and concatenated (group g at g * code_bytes / g * scale_bytes), resident
    on a device."""
    codes: "object"
    scales: "object"
    groups: int
    rows: int
    K: int

    def check(self, name: str) -> None:
        import torch
        cb, sb = packed_size(self.rows, self.K)
        for what, t, need in ((".codes", self.codes, cb * self.groups),
                              (".scales", self.scales, sb * self.groups)):
            if t.dtype != torch.uint8 or t.numel() != need or not t.is_contiguous():
                raise ValueError(f"{name}{what} must be a contiguous uint8 tensor of {need} bytes")


def pack_groups(codes: np.ndarray, scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Canonical weights [G, rows, K/2] and [G, rows, K/16] -> the
    concatenated packed arrays (nvfp4_pack per group)."""
    if codes.ndim != 3 or scales.ndim != 3 or codes.shape[0] != scales.shape[0]:
        raise ValueError("codes and scales must be [G, rows, K/2] and [G, rows, K/16]")
    parts = [pack(codes[g], scales[g]) for g in range(codes.shape[0])]
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def groups_to_device(codes: np.ndarray, scales: np.ndarray, device="cuda") -> PackedGroups:
    import torch
    G, rows, kh = codes.shape
    pc, ps = pack_groups(codes, scales)
    return PackedGroups(torch.from_numpy(pc).to(device), torch.from_numpy(ps).to(device), G, rows,
                        2 * kh)


def grouped_gemm(a: PackedOperand, b: PackedGroups, row_offsets, alpha: float = 1.0, out=None,
                 stream=None, path: int = PATH_AUTO):
    """Grouped GEMM (nvfp4_grouped_gemm, or nvfp4_grouped_gemm_with_plan for
    a forced ``path``: PATH_SKINNY, PATH_WSPLIT or PATH_TILE): rows
    row_offsets[g] .. row_offsets[g+1]-1 of A and C belong to group g, whose
    weights are b's g-th operand.  ``row_offsets`` is an int32 device tensor
    of G + 1 entries.  Returns C (M x N bfloat16)."""
    import torch
    if a.K != b.K:
        raise ValueError(f"K dimension mismatch: A has K={a.K}, B has K={b.K}")
    M, N, K = a.rows, b.rows, a.K
    if (row_offsets.dtype != torch.int32 or row_offsets.numel() != b.groups + 1
            or not row_offsets.is_contiguous() or row_offsets.device != a.codes.device):
        raise ValueError(f"row_offsets must be a contiguous int32 tensor of {b.groups + 1} "
                         "entries on A's device")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.codes.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape ({M}, {N})")
    a.check("a")
    b.check("b")
    st = lib().nvfp4_grouped_gemm_with_plan(a.codes.data_ptr(), a.scales.data_ptr(),
                                            b.codes.data_ptr(), b.scales.data_ptr(),
                                            row_offsets.data_ptr(), b.groups, float(alpha),
                                            out.data_ptr(), M, N, K, int(path),
                                            _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_grouped_gemm_with_plan(G={b.groups}, M={M}, N={N}, K={K}, "
                             f"path={path})")
    return out


def _quantize_fn(x, prefix: str) -> str:
    """The C function for x's dtype: float32 -> <prefix>, bfloat16 ->
    <prefix>_bf16 (rows of 16-byte multiples either way)."""
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 or bfloat16 tensor with unit stride along K")
    return prefix if x.dtype == torch.float32 else prefix + "_bf16"


def quantize(x, out: PackedOperand | None = None, stream=None) -> PackedOperand:
    """Quantise a 2-D fp32 or bfloat16 device tensor (rows x K, unit stride
    along K, row stride a multiple of 4 fp32 or 8 bfloat16 elements) to NVFP4
    in the packed layout (nvfp4_quantize / nvfp4_quantize_bf16); returns the
    PackedOperand (or fills ``out``)."""
    import torch
    fn = _quantize_fn(x, "nvfp4_quantize")
    rows, K = x.shape
    if out is None:
        cb, sb = packed_size(rows, K)
        out = PackedOperand(torch.empty(cb, dtype=torch.uint8, device=x.device),
                            torch.empty(sb, dtype=torch.uint8, device=x.device), rows, K)
    elif out.rows != rows or out.K != K:
        raise ValueError("out has the wrong shape")
    out.check("out")
    st = getattr(lib(), fn)(x.data_ptr(), rows, K, x.stride(0), out.codes.data_ptr(),
                            out.scales.data_ptr(), _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"{fn}(rows={rows}, K={K}, ld={x.stride(0)})")
    return out


def _activation_rows(x, b: PackedOperand, out):
    """Checks of gemm_quantized's arguments: x (M x K fp32 or bfloat16, unit
    stride along K) against B; returns (x_type, M, N, out)."""
    import torch
    if x.dtype not in (torch.float32, torch.bfloat16) or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D float32 or bfloat16 tensor with unit stride along K")
    M, K = x.shape
    if K != b.K:
        raise ValueError(f"K dimension mismatch: x has K={K}, B has K={b.K}")
    N = b.rows
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bfloat16 tensor of shape ({M}, {N})")
    b.check("b")
    return (INPUT_F32 if x.dtype == torch.float32 else INPUT_BF16), M, N, out


def gemm_quantized(x, b: PackedOperand, alpha: float = 1.0, out=None, stream=None):
    """C = gemm(quantize(x), b, alpha) in one launch (nvfp4_gemm_quantized):
    x holds 1-4 rows of fp32 or bfloat16 activations; the result equals the
    two-call form bit for bit."""
    x_type, M, N, out = _activation_rows(x, b, out)
    st = lib().nvfp4_gemm_quantized(x.data_ptr(), x_type, x.stride(0), b.codes.data_ptr(),
                                    b.scales.data_ptr(), float(alpha), out.data_ptr(), M, N, b.K,
                                    _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_gemm_quantized(M={M}, N={N}, K={b.K})")
    return out


def probe_empty(blocks: int, threads: int, stream=None) -> None:
    """Enqueue an empty kernel (nvfp4_probe_empty): a measurement aid for
    the per-call floor of a launch."""
    st = lib().nvfp4_probe_empty(blocks, threads, _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_probe_empty(blocks={blocks}, threads={threads})")


def probe_chase(next_idx, steps: int, out, stream=None) -> None:
    """One work-item follows ``next_idx`` (a device int32/uint32 tensor of a
    power-of-two length holding indices) for ``steps`` dependent loads and
    writes the last index to ``out`` (nvfp4_probe_chase): a measurement aid
    for the load latency of the cache level the array fits in."""
    st = lib().nvfp4_probe_chase(next_idx.data_ptr(), next_idx.numel(), steps, out.data_ptr(),
                                 _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_probe_chase(n={next_idx.numel()}, steps={steps})")


def probe_mfma(blocks: int, iters: int, out, stream=None) -> None:
    """Enqueue the MFMA-rate kernel (nvfp4_probe_mfma): blocks x 4 waves x
    iters x 8 fp16 MFMAs of 32 x 32 x 16; ``out`` is a float32 device tensor
    of at least blocks x 256 elements."""
    if out.numel() < blocks * 256:
        raise ValueError("out must hold blocks x 256 floats")
    st = lib().nvfp4_probe_mfma(blocks, iters, out.data_ptr(), _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_probe_mfma(blocks={blocks}, iters={iters})")


def probe_read(src, blocks: int, out, stream=None) -> None:
    """Enqueue the streaming-read kernel (nvfp4_probe_read) over all bytes
    of the device tensor ``src``."""
    st = lib().nvfp4_probe_read(src.data_ptr(), src.numel() * src.element_size(), blocks,
                                out.data_ptr(), _stream_handle(stream))
    if st:
        raise Nvfp4Error(st, f"nvfp4_probe_read(blocks={blocks})")


class Sequence:
    """A recorded sequence of NVFP4 calls replayed with one graph launch
    (nvfp4_sequence_*): record with the add_* methods (fixed buffers; the
    plans are chosen then), ``finalize()`` once, then ``launch()`` per step.
    The tensors passed in are kept referenced for the sequence's lifetime."""

    def __init__(self):
        h = _vp()
        st = lib().nvfp4_sequence_create(ctypes.byref(h))
        if st:
            raise Nvfp4Error(st, "nvfp4_sequence_create")
        self._h = h
        self._keep = []
        self.calls = 0

    def _check(self, st, what):
        if st:
            raise Nvfp4Error(st, what)
        self.calls += 1

    def add_gemm(self, a: PackedOperand, b: PackedOperand, out, alpha: float = 1.0) -> None:
        import torch
        if a.K != b.K:
            raise ValueError(f"K dimension mismatch: A has K={a.K}, B has K={b.K}")
        M, N = a.rows, b.rows
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous bfloat16 tensor of shape ({M}, {N})")
        a.check("a")
        b.check("b")
        self._keep += [a, b, out]
        self._check(lib().nvfp4_sequence_add_gemm(
            self._h, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
            b.scales.data_ptr(), float(alpha), out.data_ptr(), M, N, a.K),
            f"nvfp4_sequence_add_gemm(M={M}, N={N}, K={a.K})")

    def add_gemm_quantized(self, x, b: PackedOperand, alpha: float, out) -> None:
        """Records gemm_quantized(x, b, alpha, out)."""
        x_type, M, N, out = _activation_rows(x, b, out)
        self._keep += [x, b, out]
        self._check(lib().nvfp4_sequence_add_gemm_quantized(
            self._h, x.data_ptr(), x_type, x.stride(0), b.codes.data_ptr(), b.scales.data_ptr(),
            float(alpha), out.data_ptr(), M, N, b.K), f"nvfp4_sequence_add_gemm_quantized(M={M}, N={N})")

    def add_grouped_gemm(self, a: PackedOperand, b: "PackedGroups", row_offsets, out,
                         alpha: float = 1.0) -> None:
        import torch
        if a.K != b.K:
            raise ValueError(f"K dimension mismatch: A has K={a.K}, B has K={b.K}")
        M, N = a.rows, b.rows
        if row_offsets.dtype != torch.int32 or row_offsets.numel() != b.groups + 1:
            raise ValueError(f"row_offsets must be an int32 tensor of {b.groups + 1} entries")
        if out.dtype != torch.bfloat16 or tuple(out.shape) != (M, N) or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous bfloat16 tensor of shape ({M}, {N})")
        a.check("a")
        b.check("b")
        self._keep += [a, b, row_offsets, out]
        self._check(lib().nvfp4_sequence_add_grouped_gemm(
            self._h, a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
            b.scales.data_ptr(), row_offsets.data_ptr(), b.groups, float(alpha), out.data_ptr(),
            M, N, a.K), f"nvfp4_sequence_add_grouped_gemm(G={b.groups}, M={M}, N={N})")

    def add_quantize(self, x, out: PackedOperand) -> None:
        """Records quantize(x, out): fp32 or bfloat16 x."""
        fn = _quantize_fn(x, "nvfp4_sequence_add_quantize")
        rows, K = x.shape
        if out.rows != rows or out.K != K:
            raise ValueError("out has the wrong shape")
        out.check("out")
        self._keep += [x, out]
        self._check(getattr(lib(), fn)(
            self._h, x.data_ptr(), rows, K, x.stride(0), out.codes.data_ptr(),
            out.scales.data_ptr()), f"{fn}(rows={rows}, K={K})")

    def finalize(self) -> None:
        st = lib().nvfp4_sequence_finalize(self._h)
        if st:
            raise Nvfp4Error(st, "nvfp4_sequence_finalize")

    def launch(self, stream=None) -> None:
        st = lib().nvfp4_sequence_launch(self._h, _stream_handle(stream))
        if st:
            raise Nvfp4Error(st, "nvfp4_sequence_launch")

    def close(self) -> None:
        """Frees the graph and workspace (launches must have completed)."""
        if self._h is not None:
            lib().nvfp4_sequence_destroy(self._h)
            self._h = None
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
