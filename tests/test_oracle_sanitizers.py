"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle's C is built a second time with -fsanitize=address,undefined
-fno-sanitize-recover=all, and tests/oracle_sanitize_driver.py calls every
oracle entry point on small seeded inputs in a child process that preloads
gcc's libasan (a Python process cannot load an ASan-instrumented library
otherwise).  Any out-of-bounds access, use after free or undefined
arithmetic aborts the child with a sanitizer report."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                              timeout=30).stdout.strip()
    except (OSError, subprocess.SubprocessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's libasan is not installed")
    oracle.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, KVQ_ORACLE_SANITIZE="1",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_sanitize_driver.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert r.stdout.strip().endswith("oracle sanitize driver: ok"), report
