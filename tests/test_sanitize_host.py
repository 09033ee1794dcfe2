"""The C++ oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, g++) and run through every entry point on tiny layers
(tests/sanitize/oracle_driver.cpp): any out-of-bounds access, signed
overflow or misaligned access aborts the driver."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_ub_sanitizers():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_driver")
        cmd = [gxx, "-O1", "-g", "-std=c++17", "-pthread", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
               "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "moe_ref.cpp"),
               os.path.join(ROOT, "tests", "sanitize", "oracle_driver.cpp"), "-o", exe]
        b = subprocess.run(cmd, capture_output=True, text=True)
        if b.returncode != 0 and "asan" in (b.stderr or "").lower():
            pytest.skip("sanitizer runtime not available: " + b.stderr[-300:])
        assert b.returncode == 0, b.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
        assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
        assert "oracle driver: clean" in r.stdout
