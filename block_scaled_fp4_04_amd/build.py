"""Compile the gfx950 HIP library (libnvfp4.so) in-tree with hipcc."""
from __future__ import annotations

import hashlib
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libnvfp4.so")
SOURCES = [os.path.join(CSRC, "nvfp4_api.cpp"), os.path.join(CSRC, "nvfp4_plan.cpp"),
           os.path.join(CSRC, "nvfp4_sequence.cpp"), os.path.join(CSRC, "nvfp4_kernels.hip"), os.path.join(CSRC, "nvfp4_grouped.hip"),
           os.path.join(CSRC, "nvfp4_quantize.hip"), os.path.join(CSRC, "nvfp4_probe.hip"),
           os.path.join(CSRC, "nvfp4_noalloc.hip")]
# what the kernels and their launches are built from
KERNEL_FILES = [os.path.join(CSRC, f) for f in ("nvfp4_kernels.hip", "nvfp4_grouped.hip",
                                                "nvfp4_quantize.hip", "nvfp4_internal.h",
                                                "nvfp4_device.h", "nvfp4_quant_device.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # kernels with plain arguments get the leading ones preloaded into scalar
    # registers before their waves start (the decode-sized kernels: one
    # memory round trip less per call)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def build_id() -> str:
    """Hash of the kernel sources and compiler flags, comments and blank lines
    left out: a tuned plan table records the id of the kernels it timed."""
    h = hashlib.sha256(" ".join(HIPCC_FLAGS).encode())
    for path in KERNEL_FILES:
        text = _COMMENT.sub("", open(path).read())
        lines = [l.rstrip() for l in text.splitlines() if l.strip()]
        h.update(os.path.basename(path).encode() + b"\0" + "\n".join(lines).encode() + b"\0")
    return h.hexdigest()[:16]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-DNVFP4_BUILD_ID=\"{build_id()}\"", "-I", INCLUDE, "-I", CSRC,
           "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
