"""bench.py's command line on the host: more than one GPU is refused with a message
before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=300, cwd=ROOT)
    assert res.returncode != 0
    msg = res.stdout + res.stderr
    assert "one GPU" in msg and "--gpus 2" in msg
    assert '"metric"' not in res.stdout  # no result line
