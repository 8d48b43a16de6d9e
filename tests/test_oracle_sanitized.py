"""The oracle's pins, run against its AddressSanitizer + UndefinedBehaviorSanitizer
build (oracle/build.py, sanitize=True), in a subprocess with the ASan runtime
preloaded.  An out-of-bounds access, a use after free or undefined behaviour
(signed overflow, bad shift, misaligned access ...) anywhere the pins reach
aborts the run."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc's ASan runtime is not available")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=rt, ORACLE_LIB=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = ("import ctypes, oracle; "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'), 'ASan runtime not loaded'; "
             "assert oracle.lib()._name == __import__('os').environ['ORACLE_LIB']; print('asan-active')")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "asan-active" in r.stdout, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_compress_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
