"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code only).

A child process loads the sanitized build of oracle/ (libasan preloaded, since the interpreter is
not instrumented) and runs the oracle's stream, corrupt-stream, Rice and transform tests; any
out-of-bounds access, use after free, signed overflow or other undefined behaviour aborts it.  The
whole CPU suite runs the same way with the command in oracle/__init__.py.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    except OSError:
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_tests_pass_under_sanitizers():
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    import oracle
    oracle.build(sanitize=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["HQO_SANITIZE"] = "1"
    tests = ["tests/test_oracle_corrupt.py", "tests/test_oracle_rice.py", "tests/test_oracle_rht.py",
             "tests/test_oracle_golden.py", "tests/test_encode_bound.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
