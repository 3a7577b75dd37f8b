"""Host check of the state phase's row assignment (dot_rows / dot_row in
csrc/dh_phases.h): for many shapes and grids, in both block widths, every row of
[W1_S; W_hh] is computed exactly once, by the block that owns it, u rows first in
each wave, and no wave holds more rows than the LDS cache has slots for.  The header
is compiled by hipcc into a host program (no GPU is used)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "causal_draft_correction_amd", "csrc")

PROG = r"""
#include "dh_phases.h"
#include <cstdio>
#include <vector>
using namespace DH_NS;
int main()
{
    int bad = 0, grouped = 0;
    const int rs[] = {16, 32, 64, 256, 512, 1024}, hs[] = {64, 128, 256, 1024, 1536, 2048};
    const int gs[] = {1, 3, 7, 16, 64, 100, 128, 255, 256, 304, 1024};
    for (int group = 0; group < 2; ++group)
        for (int r : rs)
            for (int h : hs)
                for (int nblk : gs) {
                    const int R = r + 3 * h, cap = state_rows_per_wave(r, h, nblk);
                    std::vector<int> seen(R, 0);
                    for (int blk = 0; blk < nblk; ++blk) {
                        const DotRows d = dot_rows(r, R, blk, nblk, group != 0);
                        grouped += d.rg > 1;
                        for (int w = 0; w < NWAVE; ++w) {
                            const int n = dot_rows_of(d, w), nu = dot_u_rows(d, w);
                            bad += n > cap;
                            for (int k = 0; k < n; ++k) {
                                const int m = dot_row(d, w, k);
                                if (m < 0 || m >= R) { ++bad; continue; }
                                bad += (k < nu) != (m < r);
                                bad += m % nblk != blk;
                                ++seen[m];
                            }
                            bad += dot_row(d, w, n) != -1;
                        }
                    }
                    for (int m = 0; m < R; ++m)
                        bad += seen[m] != 1;
                }
    // the 8B head on 256 four-wave blocks: one u row on wave 0, four q rows on each other wave
    if (NWAVE == 4) {
        const DotRows d = dot_rows(256, 256 + 3 * 1024, 7, 256);
        bad += !(d.rg == 4 && dot_rows_of(d, 0) == 1 && dot_u_rows(d, 0) == 1 && dot_rows_of(d, 1) == 4 &&
                 dot_rows_of(d, 2) == 4 && dot_rows_of(d, 3) == 4);
    }
    std::printf("bad %d grouped %d\n", bad, grouped);
    return bad != 0;
}
"""


def _hipcc():
    return shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)


@pytest.mark.parametrize("nt", [256, 512])
def test_dot_rows_cover_every_row_once(tmp_path, nt):
    cc = _hipcc()
    if not cc:
        pytest.skip("hipcc not available")
    src = tmp_path / "dot_rows_check.hip"
    src.write_text(PROG)
    exe = tmp_path / "dot_rows_check"
    cmd = [cc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-DDH_NT=%d" % nt, "-DDH_NS=dhc%d" % nt,
           "-I", CSRC, str(src), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("bad 0 ")
