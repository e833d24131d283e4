"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc), every pin run against it in a child process: an out-of-bounds access,
a use after free, a signed overflow or a misaligned access anywhere on the
pinned paths aborts the child and fails the test.  CPU only."""
import os
import subprocess
import sys
import tempfile

import pytest

from oracle.oracle import SRC, build_oracle

_RUN = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from oracle.oracle import load_oracle
import oracle_pins
lib = load_oracle({lib!r})
for name, pin in oracle_pins.ALL_PINS.items():
    fails = pin(lib)
    if fails:
        print("pin", name, "failed:", fails[0][:200])
        sys.exit(3)
print("all pins clean")
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's AddressSanitizer runtime is not installed")
def test_pins_pass_under_asan_and_ubsan():
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests_dir)
    with tempfile.TemporaryDirectory() as d:
        lib = build_oracle(out=os.path.join(d, "liboracle_san.so"),
                           extra_flags=["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                        "-fno-sanitize-recover=all"])
        env = dict(os.environ, LD_PRELOAD=_runtime("libasan.so"),
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        res = subprocess.run([sys.executable, "-c", _RUN.format(root=root, tests=tests_dir, lib=lib)],
                             capture_output=True, text=True, timeout=600, env=env)
        report = (res.stdout + res.stderr)[-3000:]
        assert res.returncode == 0, report
        assert "all pins clean" in res.stdout
        assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, report
