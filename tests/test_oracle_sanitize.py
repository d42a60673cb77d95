"""The oracle's pins on an AddressSanitizer + UndefinedBehaviorSanitizer build
of the oracle (CPU only).

The oracle is C++ that every parity claim rests on, so an out-of-bounds read,
a signed overflow or a bad shift in it must not go unseen.  This builds
lqref.cpp with -fsanitize=address,undefined (no recovery: the first report
aborts), then runs every pin of the oracle (exact-arithmetic pins, the
quantizer's and the integer-dot path's) in a child process with the ASan
runtime preloaded (Python itself is not instrumented).  A sanitizer report
fails the test with its text.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lqref.cpp")

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from oracle import lqref
from tests.test_oracle_pins import ALL_PINS
from tests.test_oracle_quant import QUANT_PINS
from tests.test_oracle_q8act import Q8ACT_PINS
o = lqref.Oracle({so!r})
pins = ALL_PINS + QUANT_PINS + Q8ACT_PINS
for pin in pins:
    pin(o)
print("pins passed:", len(pins), flush=True)
"""


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None or _runtime("libubsan.so") is None:
        pytest.skip("the host compiler has no sanitizer runtimes")
    so = str(tmp_path / "liblqref_sanitized.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-o", so, SRC], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, so=so)], env=env, capture_output=True,
                       text=True, timeout=600)
    report = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, report
    assert "pins passed:" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
