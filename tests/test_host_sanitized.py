"""The C-ABI library with its host code built under AddressSanitizer and
UndefinedBehaviorSanitizer (device code unchanged; each -fsanitize= goes to the
host pass only): the host-side ABI tests (argument validation, workspace
sizing, config checks, parameter counts, NULL handles) run against that build
in a child process, so a host-side overrun or undefined behaviour in the entry
points fails this test.  No GPU is used."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from causal_draft_correction_amd import build as hipbuild  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _runtime():
    c = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return c[-1] if c else None


@pytest.mark.skipif(_runtime() is None, reason="clang ASan runtime not found")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    cc = hipbuild.hipcc()
    flags = [f for f in hipbuild.FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN
    objs = [str(tmp_path / u.replace(".hip", ".o")) for u in hipbuild.UNITS]
    jobs = [[cc] + flags + ["-c", os.path.join(hipbuild.SRC_DIR, u), "-o", o] for u, o in zip(hipbuild.UNITS, objs)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs):
            assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libdomino_head_san.so")
    r = subprocess.run([cc, "--offload-arch=" + hipbuild.ARCH, "-shared", "-fPIC", "-shared-libsan"] + SAN[:4] +
                       objs + ["-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, DOMINO_LIB=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    probe = ("import ctypes, causal_draft_correction_amd as d; d.load_library(); "
             "print(d.LIB_PATH, hasattr(ctypes.CDLL(None), '__asan_init'))")
    out = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0 and out.stdout.split() == [lib, "True"], out.stdout + out.stderr[-2000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, tail
    assert " passed" in res.stdout, tail
