"""Builds libdomino_head.so (HIP, gfx950) in the package directory."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC_DIR = os.path.join(HERE, "csrc")
MAIN_SRC = os.path.join(SRC_DIR, "domino_head.hip")
RES_SRC = os.path.join(SRC_DIR, "domino_head_res.hip")
BAT_SRC = os.path.join(SRC_DIR, "domino_head_bat.hip")
VER_SRC = os.path.join(SRC_DIR, "domino_verify.hip")
LIB = os.path.join(HERE, "libdomino_head.so")
ARCH = "gfx950"


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


def build(verbose: bool = False) -> str:
    """Compile the library for gfx950.  Packed-fp32 instructions are disabled."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", MAIN_SRC, RES_SRC, BAT_SRC, VER_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + errs)
    if verbose and errs.strip():
        print(errs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
