"""The per-phase tracing build (libdomino_trace.so) on the device: the phases the
tracer reports for the resident B = 1 kernel and the batched kernel cover each
position, and the instrumented library drafts the same tokens as the product
library.  Runs the tracer in a child process (it loads the instrumented library in
place of the product one).  The child starts its kernels with ordinary launches: while
this test process, which has made cooperative launches, is alive, a cooperative launch
from another process on the same GPU is refused (hipErrorIllegalState).  Its grid is one
block per compute unit and this process is idle meanwhile, so every block is resident."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRACE_LIB = os.path.join(ROOT, "causal_draft_correction_amd", "libdomino_trace.so")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(TRACE_LIB):
        pytest.skip("libdomino_trace.so is not built")


CHILD = r"""
import json, sys
import numpy as np, torch
sys.path.insert(0, %(root)r)
from causal_draft_correction_amd import phase_trace
import causal_draft_correction_amd as dca
import domino_synth as ds
res = phase_trace.run([%(wl)r], persistent=True, plain_launch=True)
r = res[%(wl)r]
# the instrumented library drafts like the product one: compare with the oracle's first token
w, inp = ds.make_workload(%(wl)r)
head = dca.DominoHead(dca.head_weights_to_device(w), K=w.shape.K, max_batch=inp.H.shape[0], fold_embedding=True,
                      exec_mode=dca.EXEC_PLAIN_LAUNCH)
out = head.draft(dca.device_tensor(inp.H), dca.device_tensor(inp.L_base), dca.device_tensor(inp.last_tok))
torch.cuda.synchronize()
r["tokens0"] = out["tokens"][:, 0].cpu().numpy().tolist()
print("RESULT " + json.dumps(r))
"""


@pytest.mark.parametrize("wl", ["qwen3_8b_b1", "qwen3_8b_b32"])
def test_phase_trace_reports_every_phase(wl):
    res = subprocess.run([sys.executable, "-c", CHILD % {"root": ROOT, "wl": wl}], capture_output=True, text=True,
                         timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    line = [l for l in res.stdout.splitlines() if l.startswith("RESULT ")][-1]
    r = json.loads(line[len("RESULT "):])
    mid = r["positions_1_to_14_median"]
    # every phase took a positive time and the phases add up to the position
    # (the dots_, exchange_ and gates_ entries split state_dots, argmax_exchange and gru_gates)
    parts = {k: v[0] for k, v in mid.items()
             if k != "position" and not k.startswith(("dots_", "exchange_", "gates_")) and k != "mark_cost"}
    assert all(v > 0 for v in parts.values()), parts
    assert 0.8 * mid["position"][0] <= sum(parts.values()) <= 1.2 * mid["position"][0], (parts, mid["position"])
    # the kernel spans the prologue and 16 positions
    assert r["kernel_us"] > r["prologue"]["prologue"][0] + 14 * mid["position"][0] * 0.8
    assert r["call_us"] >= 0.9 * r["kernel_us"]
    # the first drafted tokens equal the oracle's where the oracle's gap is clear
    import domino_synth as ds
    import oracle
    w, inp = ds.make_workload(wl)
    rows = [0]
    o = oracle.draft(w, inp.H[rows], inp.L_base[rows], inp.last_tok[rows])
    if o["gap"][0, 0] > 5e-2:
        assert r["tokens0"][0] == int(o["tokens"][0, 0])
