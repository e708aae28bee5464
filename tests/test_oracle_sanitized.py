"""Every oracle pin again, with the C oracle built under AddressSanitizer and
UndefinedBehaviorSanitizer (gcc, host code only; no GPU).

The instrumented library is loaded into a child interpreter that has the
ASan runtime preloaded (a sanitized shared object cannot be loaded into an
uninstrumented process otherwise).  Any out-of-bounds access, use after free
or undefined behaviour (signed overflow, bad shift, misaligned load, ...)
aborts the child, and the test fails with its report.
"""
import os
import subprocess
import sys

import pytest

import oracle.build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

SAN_FLAGS = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g")

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load_library({lib!r})
for pin in ALL_PINS:
    pin(lib)
    print("pin ok", pin.__name__, flush=True)
print("ALL", len(ALL_PINS), flush=True)
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's ASan runtime is not installed")
    lib = str(tmp_path / "libmoe_oracle_san.so")
    obuild.build(out=lib, extra_flags=SAN_FLAGS)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    # CPython keeps its interned objects to the end: leak reports are noise
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout[-2000:] + "\n" + r.stderr[-6000:])
    assert r.returncode == 0, tail
    assert "ALL" in r.stdout, tail
    for word in ("AddressSanitizer", "runtime error"):
        assert word not in r.stderr, tail
