"""The oracle's C code built with AddressSanitizer and UndefinedBehaviorSanitizer (host code, gcc),
run through every pin (CPU only).  An out-of-bounds access, a use of freed memory or undefined
behaviour in the oracle stops the run with a report instead of passing silently."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

RUN_PINS = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
lib = oracle.load_variant({so!r})
for pin in oracle_pins.ALL_PINS:
    pin(lib=lib)
    print("ok", pin.__name__, flush=True)
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    so = tmp_path / "libssd_oracle_san.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                           "-o", str(so), SRC, "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    code = RUN_PINS.format(root=ROOT, tests=HERE, so=str(so))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    from oracle_pins import ALL_PINS
    assert out.count("ok pin_") == len(ALL_PINS), out[-2000:]
