"""GPU parity of the greedy verify step (through the C ABI) against the oracle.

The step is integer work on float32 inputs (argmax decisions, prefix match), so
every output must equal the oracle's bit for bit.
"""
import numpy as np
import pytest
import torch

import causal_draft_correction_amd as dca
import domino_synth as ds
import oracle
from gpu_common import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dca.load_library()


def run_gpu(logits, draft, want_target=True):
    lg = dca.device_tensor(np.ascontiguousarray(logits, np.float32))
    dr = dca.device_tensor(np.ascontiguousarray(draft, np.int32))
    out = dca.verify(lg, dr, want_target=want_target)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check(logits, draft, label):
    o = oracle.verify(logits, draft)
    g = run_gpu(logits, draft)
    for k in ("target", "accept", "next"):
        assert np.array_equal(o[k], g[k]), "%s: %s differs" % (label, k)
    g2 = run_gpu(logits, draft, want_target=False)
    assert np.array_equal(g2["accept"], o["accept"]) and np.array_equal(g2["next"], o["next"])
    log("%s: accept %s" % (label, o["accept"][:8].tolist()))
    return o


def plant_specials(lg):
    """Ties, NaN and +-0 spread over the whole row, so they straddle however the
    row is split between blocks."""
    B, K1, V = lg.shape
    ties = np.unique(np.linspace(V // 7, V - 1, 9).astype(int))
    lg[0, 0, ties] = 1e3                  # equal maxima all along the row: the lowest index wins
    lg[0, 1, [2 * V // 3, V // 3]] = np.nan   # the first NaN wins
    lg[0, 2, V - 3] = np.inf
    lg[0, 2, 1] = 5e3                     # +inf late in the row beats a large number early
    lg[0, 3] = 0.0
    lg[0, 3, :V // 2] = -0.0              # a row of +-0: index 0
    lg[0, 4] = -np.inf                    # a row of -inf: index 0
    lg[0, 5, V - 1] = 2e3                 # the last index
    if B > 1:
        lg[1, 0, V - 1] = np.nan          # NaN on the last element


@pytest.mark.parametrize("B,K,V", [(3, 16, 5003), (3, 16, 8192), (5, 7, 40000), (2, 1, 9), (4, 16, 1)])
def test_verify_matches_oracle(B, K, V):
    vi = ds.make_verify_inputs(B, K, V, (22, B, K, V))
    lg = vi.logits.copy()
    if V > 4 and K >= 5:
        plant_specials(lg)
    draft = vi.draft.copy()
    draft[-1, 0] = -1                     # an invalid draft token never matches
    check(lg, draft, "B=%d K=%d V=%d" % (B, K, V))


def test_verify_all_accepted_and_zero_rows():
    vi = ds.make_verify_inputs(6, 16, 3001, (23, 0))
    o = check(vi.logits, vi.planted[:, :16], "all accepted")
    assert (o["accept"] == 16).all() and np.array_equal(o["next"], vi.planted[:, 16])
    lg = dca.device_tensor(vi.logits[:0].copy())
    dr = dca.device_tensor(vi.draft[:0].copy())
    out = dca.verify(lg, dr)  # B = 0: nothing launched
    torch.cuda.synchronize()
    assert out["accept"].numel() == 0


@pytest.mark.parametrize("B", [1, 32])
def test_verify_full_vocabulary(B):
    """V = 151936 (the 8B head's vocabulary) at B = 1 and at B = 32, the launch
    configuration the benchmark times."""
    vi = ds.make_verify_inputs(B, 16, 151936, (24, B))
    lg = vi.logits
    plant_specials(lg)
    o = check(lg, vi.draft, "full V B=%d" % B)
    if B == 32:
        assert (o["accept"] == np.minimum(vi.k, 16))[1:].all()
