"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the C
oracle is rebuilt with both and every GEMM and quantiser pin runs against it
in a child process (the sanitizer runtimes must be loaded before Python).
A memory error or an undefined operation aborts the child, which fails the
test; no GPU is involved."""
import os
import shutil
import subprocess
import sys

import pytest

from oracle import oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {here!r})
import oracle_pins as pins, quant_pins as qp
from oracle import oracle as orc
o = orc.load({lib!r})
bad = {{k: v[:2] for k, v in pins.run_all(o, quick=True).items() if v}}
for p in qp.ALL_QUANT_PINS:
    f = p(o)
    if f:
        bad[p.__name__] = f[:2]
print("SANITIZED-PINS", len(pins.ALL_PINS) + len(qp.ALL_QUANT_PINS), "failed:", bad, flush=True)
sys.exit(1 if bad else 0)
"""


def _runtime(name: str) -> str | None:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = orc.build(str(tmp_path / "liboracle_sanitized.so"),
                    extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                                 "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ, LD_PRELOAD=f"{asan} {ubsan}", ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, here=HERE, lib=lib)],
                       capture_output=True, text=True, env=env, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "SANITIZED-PINS" in r.stdout and "failed: {}" in r.stdout, tail
