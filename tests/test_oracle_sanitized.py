"""The oracle's pins and its mutation test, run again on a build of oracle.c
with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU only).  Every
oracle function the pins call, on every pin's inputs (empty shards, -inf, NaN,
+inf, K = cols, bf16 rows), runs without a memory or undefined-behaviour
report, and each planted mistake is still caught."""
import os
import shutil
import subprocess
import sys

import pytest

from oracle.build import SANITIZE_ENV

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _libasan():
    cc = shutil.which("gcc")
    if cc is None:
        return None
    path = subprocess.run([cc, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pins_and_mutants_under_sanitizers():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc's libasan is not available")
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **{SANITIZE_ENV: "1"})
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(HERE, "test_oracle.py"), os.path.join(HERE, "test_oracle_mutants.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out, out[-2000:]
