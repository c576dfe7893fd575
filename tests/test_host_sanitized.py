"""The host half of the library under AddressSanitizer and
UndefinedBehaviorSanitizer: the C ABI's argument checks, the packer, the
plan rules, the plan-table reader and the sequence bookkeeping are rebuilt
with g++ and both sanitizers (the kernel launches replaced by stubs that
return an error; these tests never launch), and the CPU ABI and plan-table
tests run against that build in a child process with the sanitizer runtimes
preloaded.  A memory error in the library's own allocations or stack, or an
undefined operation, aborts the child.  (Buffers that the tests pass in come
from Python's allocator, which AddressSanitizer does not instrument: writes
past them are not seen here; the packer's bounds are pinned by the layout
tests instead.)"""
import os
import shutil
import subprocess
import sys

import pytest

import block_scaled_fp4_04_amd as nv
from block_scaled_fp4_04_amd import build as nvbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

# Stand-ins for the device side (kernel launches and their workspace sizes).
STUBS = r"""
#include "nvfp4_internal.h"
namespace nvfp4 {
hipError_t launch_tile(int, const GemmArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_wsplit(int, const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_skinny(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemv(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_grouped(const GroupedArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_grouped_wsplit(const GroupedArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_grouped_tile(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quantize(const QuantArgs&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemv_quant(const GemvQuantArgs&, hipStream_t) { return hipErrorInvalidValue; }
size_t tile_partial_floats(int, const GemmArgs&) { return 0; }
size_t tile_counters(int, const GemmArgs&) { return 0; }
size_t skinny_flagged_words(const GemmArgs&) { return 0; }
size_t skinny_counters(const GemmArgs&) { return 0; }
size_t wsplit_partial_floats(int, const GemmArgs&) { return 0; }
int resident_tiles(int, int) { return 0; }
hipError_t take_device_flags(uint32_t* flags) { *flags = 0; return hipErrorInvalidValue; }
int noalloc_setup(int) { return 4; }
}
extern "C" int nvfp4_probe_empty(int64_t, int64_t, void*) { return 1; }
extern "C" int nvfp4_probe_chase(const uint32_t*, int64_t, int64_t, uint32_t*, void*) { return 1; }
extern "C" int nvfp4_probe_mfma(int64_t, int64_t, float*, void*) { return 1; }
extern "C" int nvfp4_probe_read(const void*, int64_t, int64_t, uint32_t*, void*) { return 1; }
extern "C" int nvfp4_gemm_noalloc(const void*, const void*, const void*, const void*, float, void*,
                                  int64_t, int64_t, int64_t, void*) { return 1; }
extern "C" int nvfp4_noalloc_scratch_bytes(int64_t, int64_t, int64_t, size_t*) { return 1; }
"""

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {here!r})
import block_scaled_fp4_04_amd as nv
nv.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      {abi!r}, {table!r}]))
"""


def _runtime(name: str) -> str | None:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs gcc and g++")
def test_host_library_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    hip = os.path.join(ROCM, "lib", "libamdhip64.so")
    if not asan or not ubsan or not os.path.exists(hip):
        pytest.skip("sanitizer runtimes or the HIP runtime not installed")
    stubs = tmp_path / "device_stubs.cpp"
    stubs.write_text(STUBS)
    lib = str(tmp_path / "libnvfp4_host_sanitized.so")
    host = [os.path.join(nvbuild.CSRC, f) for f in ("nvfp4_api.cpp", "nvfp4_plan.cpp",
                                                    "nvfp4_sequence.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           f"-DNVFP4_BUILD_ID=\"{nvbuild.build_id()}\"", "-I", os.path.join(ROCM, "include"),
           "-I", nvbuild.INCLUDE, "-I", nvbuild.CSRC, *host, str(stubs), "-o", lib,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    child = CHILD.format(root=ROOT, here=HERE, lib=lib,
                         abi=os.path.join(HERE, "test_abi.py"),
                         table=os.path.join(HERE, "test_plan_table.py"))
    r = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env,
                       timeout=600, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
    assert nv.LIB_PATH != lib  # the parent process keeps the real library
