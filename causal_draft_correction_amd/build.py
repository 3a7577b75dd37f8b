"""Builds libdomino_head.so (HIP, gfx950) in the package directory, and beside it
libdomino_trace.so: the same library with the persistent kernels' phase hooks
recording device timestamps (read by phase_trace.py; never loaded otherwise)."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_DIR = os.path.join(HERE, "csrc")
UNITS = ["domino_head.hip", "domino_head_res.hip", "domino_head_bat.hip", "domino_head_rb.hip", "domino_verify.hip"]
LIB = os.path.join(HERE, "libdomino_head.so")
# the instrumented library: these units replace domino_head_res.hip and domino_head_rb.hip
TRACE_UNITS = ["trace/trace_res.hip", "trace/trace_rb.hip"]
TRACE_REPLACES = ["domino_head_res.hip", "domino_head_rb.hip"]
TRACE_LIB = os.path.join(HERE, "libdomino_trace.so")
ARCH = "gfx950"
# packed-fp32 instructions are disabled in all device code
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    out = []
    for root, _, files in os.walk(SRC_DIR):
        out += [os.path.join(root, f) for f in files if f.endswith((".hip", ".h"))]
    out.append(os.path.join(os.path.dirname(HERE), "include", "domino_head.h"))
    return out


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in sources())


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + errs)
    return errs


def build(verbose: bool = False, trace: bool = True) -> str:
    """Compile each translation unit for gfx950 (in parallel), then link the library
    (and, with `trace`, the instrumented library from the same objects)."""
    cc = hipcc()
    units = UNITS + (TRACE_UNITS if trace else [])
    with tempfile.TemporaryDirectory(prefix="domino_build_") as tmpdir:
        obj = {u: os.path.join(tmpdir, os.path.basename(u).replace(".hip", ".o")) for u in units}
        jobs = [[cc] + FLAGS + ["-c", os.path.join(SRC_DIR, u), "-o", obj[u]] for u in units]
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            errs = list(ex.map(_run, jobs))
        links = [(LIB, [obj[u] for u in UNITS])]
        if trace:
            links.append((TRACE_LIB, [obj[u] for u in UNITS if u not in TRACE_REPLACES] +
                          [obj[u] for u in TRACE_UNITS]))
        for lib, objs in links:
            tmp = lib + ".tmp%d" % os.getpid()
            errs.append(_run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp]))
            os.replace(tmp, lib)
    if verbose and any(e.strip() for e in errs):
        print("\n".join(e for e in errs if e.strip()))
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
