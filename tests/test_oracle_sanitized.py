"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: all of
its pins and the torch cross-check in a child process
with the sanitized build loaded and gcc's ASan runtime preloaded.  Any
out-of-bounds access, use of freed memory or undefined operation in the C
oracle aborts the child and fails the test.  CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_pins_under_asan_and_ubsan():
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    sys.path.insert(0, ROOT)
    import oracle
    lib = oracle.build_sanitized()
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's libasan not found")
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py"),
         os.path.join(ROOT, "tests", "test_oracle_torch_crosscheck.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
