"""The allocation-free verify entry point (domino_verify_noalloc, static device
scratch instead of a workspace) against domino_verify with a workspace, called
through the C ABI: two calls in a row, the second smaller, then the largest
size the static scratch allows.  Integer outputs, so bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import causal_draft_correction_amd as dca
import domino_synth as ds

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return dca.load_library()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _outs(B, K):
    return {"target": torch.full((B, K + 1), -5, dtype=torch.int32, device="cuda"),
            "accept": torch.full((B,), -5, dtype=torch.int32, device="cuda"),
            "next": torch.full((B,), -5, dtype=torch.int32, device="cuda")}


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _both(lib, lg, dr):
    B, K = dr.shape
    V = lg.shape[2]
    n = ctypes.c_size_t()
    assert lib.domino_verify_workspace_size(B, K, V, ctypes.byref(n)) == 0
    ws = torch.empty(max(int(n.value), 16), dtype=torch.uint8, device="cuda")
    a, b = _outs(B, K), _outs(B, K)
    assert lib.domino_verify(B, K, V, _p(lg), _p(dr), _p(ws), ws.numel(), _p(a["target"]), _p(a["accept"]),
                             _p(a["next"]), _stream()) == 0
    assert lib.domino_verify_noalloc(B, K, V, _p(lg), _p(dr), _p(b["target"]), _p(b["accept"]), _p(b["next"]),
                                     _stream()) == 0
    torch.cuda.synchronize()
    for k in ("target", "accept", "next"):
        assert torch.equal(a[k], b[k]), k
    return b


def test_noalloc_verify_equals_workspace_verify_on_consecutive_calls(lib):
    # first call: many rows over a large vocabulary; second: fewer rows, smaller K and V
    # (the static scratch keeps the first call's keys; the second must not read them)
    for (B, K, V), key in (((48, 16, 151936), (21, 0)), ((5, 7, 30011), (21, 1))):
        vi = ds.make_verify_inputs(B, K, V, key)
        lg, dr = dca.device_tensor(vi.logits), dca.device_tensor(vi.draft)
        got = _both(lib, lg, dr)
        assert np.array_equal(got["accept"].cpu().numpy(), np.minimum(vi.k, K))
    # no target row stored: accept and next still agree
    out = _outs(B, K)
    assert lib.domino_verify_noalloc(B, K, V, _p(lg), _p(dr), None, _p(out["accept"]), _p(out["next"]),
                                     _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(out["accept"].cpu().numpy(), np.minimum(vi.k, K))
    assert int(out["target"].min()) == -5  # untouched


def test_noalloc_verify_at_the_largest_scratch(lib):
    K, V = 16, 1024
    B = (SCRATCH_BYTES // 8) // (K + 1)  # one key per row (V below one chunk)
    n = ctypes.c_size_t()
    assert lib.domino_verify_workspace_size(B, K, V, ctypes.byref(n)) == 0 and n.value <= SCRATCH_BYTES
    g = torch.Generator(device="cuda").manual_seed(1234)
    lg = torch.randn((B, K + 1, V), generator=g, device="cuda")
    dr = torch.randint(0, V, (B, K), generator=g, device="cuda", dtype=torch.int32)
    # make most rows accept a few tokens: copy the row argmax into the draft for a random prefix
    am = lg.argmax(dim=2).to(torch.int32)
    k = torch.randint(0, K + 1, (B,), generator=g, device="cuda")
    keep = torch.arange(K, device="cuda")[None, :] < k[:, None]
    dr = torch.where(keep, am[:, :K], dr).contiguous()
    _both(lib, lg, dr)


def test_noalloc_verify_refuses_more_than_its_scratch(lib):
    K, V = 16, 1024
    B = (SCRATCH_BYTES // 8) // (K + 1) + 1
    n = ctypes.c_size_t()
    assert lib.domino_verify_workspace_size(B, K, V, ctypes.byref(n)) == 0 and n.value > SCRATCH_BYTES
    # refused on the host before any device work (the pointers are never touched)
    fake = ctypes.c_void_p(256)
    rc = lib.domino_verify_noalloc(B, K, V, fake, fake, None, fake, fake, None)
    assert rc == -2
    assert b"static buffer" in lib.domino_last_error()
    assert lib.domino_verify_noalloc(0, K, V, None, None, None, None, None, None) == 0
