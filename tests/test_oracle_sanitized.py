"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle.c walks variable-length samples with plain pointer arithmetic, so its
pins are run once more in a child process against a build of the same source
with -fsanitize=address,undefined (the child preloads gcc's ASan runtime,
since the Python interpreter itself is not instrumented).  Any sanitizer
report or a failing pin fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    libasan = _runtime("libasan.so")
    if libasan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-o", lib, SRC, "-lm"])
    env = dict(os.environ, LD_PRELOAD=libasan, MPB_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-x",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_splitk_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_bwd_pins.py"),
           "-k", "not autograd"]
    r = subprocess.run(cmd, env=env, capture_output=True, text=True, cwd=ROOT, timeout=900)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    assert " passed" in r.stdout
