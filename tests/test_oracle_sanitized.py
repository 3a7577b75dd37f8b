"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only, gcc): the oracle pins run against that build in a child
process, so any out-of-bounds access, use after free, signed overflow or other
undefined behaviour in the oracle aborts the run and fails this test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(shutil.which("gcc") is None or _libasan() is None, reason="gcc with libasan needed")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
                    "-ffp-contract=off", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "domino_oracle.c"), "-o", lib, "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=_libasan(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    # the child loads the sanitized build, with the ASan runtime in the process
    probe = ("import ctypes, oracle; oracle.max_threads(); "
             "print(oracle.lib_path(), hasattr(ctypes.CDLL(None), '__asan_init'))")
    out = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0 and out.stdout.split() == [lib, "True"], out.stdout + out.stderr[-2000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
    assert " passed" in res.stdout, tail
