"""GPU parity of the Markov head (DOMINO_MARKOV) against the fp64 oracle.

The news.sig.ai article (section 从Domino看DSpark) names a Markov head beside
the recurrent one without a formula.  Reading (the oracle's): position p is
conditioned on the preceding token alone, S_p = GRU(E[x_p], 0).  The device
gathers W1_S S_p from a per-token table filled at create.

Protocols: free running up to the first token divergence (which must sit at an
oracle top-1/top-2 gap <= 5e-2), and teacher forcing with the oracle's own
draft (every position compares).  Tolerances: L_final 2e-2 abs (1e-4 for the
float32 tiny head), u 1e-4 abs, tokens identical where the oracle gap > 5e-2.
"""
import numpy as np
import pytest
import torch

import causal_draft_correction_amd as dca
import domino_synth as ds
import oracle
from gpu_common import GAP_TOL, gpu_draft, log

pytestmark = pytest.mark.gpu

LF_TOL = 2e-2
U_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dca.load_library()


def markov_head(w, max_batch, exec_mode=dca.EXEC_AUTO, K=None, lbase_bf16=False):
    return dca.DominoHead(dca.head_weights_to_device(w), K=K or w.shape.K, max_batch=max_batch, exec_mode=exec_mode,
                          lbase_bf16=lbase_bf16, markov=True)


def check_free_running(o, g, lf_tol=LF_TOL, orows=None):
    n, K = g["tokens"].shape
    orows = list(range(n)) if orows is None else list(orows)
    diverged = 0
    for gi, oi in enumerate(orows):
        bad = np.flatnonzero(o["tokens"][oi] != g["tokens"][gi])
        j = int(bad[0]) if len(bad) else K
        if j < K:
            diverged += 1
            assert o["gap"][oi, j] <= GAP_TOL, "row %d: token %d differs at oracle gap %g" % (oi, j, o["gap"][oi, j])
        upto = min(j + 1, K)
        if "L_final" in g:
            err = np.abs(o["L_final"][oi, :upto] - g["L_final"][gi, :upto]).max()
            assert err <= lf_tol, "row %d: L_final max abs err %g" % (oi, err)
        if "u" in g:
            err = np.abs(o["u"][oi, :upto] - g["u"][gi, :upto]).max()
            assert err <= U_TOL, "row %d: u max abs err %g" % (oi, err)
    return diverged


def check_teacher_forced(o, g, lf_tol=LF_TOL, orows=None):
    n = g["tokens"].shape[0]
    orows = list(range(n)) if orows is None else list(orows)
    sure = o["gap"][orows] > GAP_TOL
    assert np.array_equal(o["tokens"][orows][sure], g["tokens"][sure]), "tokens differ where the oracle gap > 5e-2"
    if "L_final" in g:
        err = np.abs(o["L_final"][orows] - g["L_final"]).max()
        assert err <= lf_tol, "L_final max abs err %g" % err
    if "u" in g:
        err = np.abs(o["u"][orows] - g["u"]).max()
        assert err <= U_TOL, "u max abs err %g" % err


def both_protocols(w, inp, head, lf_tol=LF_TOL, label=""):
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, markov=True)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    assert flags == 0
    assert "S" not in g
    div = check_free_running(o, g, lf_tol)
    ot = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=o["tokens"], markov=True)
    gt, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=o["tokens"])
    assert flags == 0
    check_teacher_forced(ot, gt, lf_tol)
    log("%s: diverged=%d, L_final err tf=%.3g, u err tf=%.3g" % (
        label, div, np.abs(ot["L_final"] - gt["L_final"]).max(), np.abs(ot["u"] - gt["u"]).max()))
    return o, g


def test_markov_tiny_fp32_head():
    """Float32 weights take the step launches; a forced persistent launch is refused."""
    w, inp = ds.make_workload("tiny")
    head = markov_head(w, 1)
    assert not head.exec_info(1)["persistent"]
    both_protocols(w, inp, head, lf_tol=1e-4, label="markov tiny")
    with pytest.raises(dca.DominoError):
        markov_head(w, 1, dca.EXEC_PERSISTENT).draft(dca.device_tensor(inp.H), dca.device_tensor(inp.L_base),
                                                     dca.device_tensor(inp.last_tok))


@pytest.mark.parametrize("K", [16, 5])
def test_markov_ragged_bf16(K):
    """r = 64 (vector-unit W2 launches); V, d, h divide no tile; GRU-sensitive weights."""
    sh = ds.HeadShape(d=520, h=136, r=64, V=5003, K=K, wdtype="bf16")
    w = ds.make_weights(sh, (9, 60), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 61), sigma=0.5, peak="none")
    both_protocols(w, inp, markov_head(w, 4), label="markov ragged K=%d" % K)


@pytest.mark.parametrize("V,B", [(5003, 1), (5003, 3), (5003, 8), (160000, 2)])
def test_markov_resident_matches_oracle_and_step_launches(V, B):
    """bf16, r = 256, B <= 8: the resident-W2 Markov kernel against the oracle, run to
    run, and bitwise against the step launches (same u and W2 arithmetic).  V = 160000
    puts tiles beyond the register share into LDS."""
    sh = ds.HeadShape(d=256, h=128, r=256, V=V, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 62), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 63), sigma=0.5, peak="none")
    head = markov_head(w, 8)
    info = head.exec_info(B)
    assert info["persistent"] and info["w2_resident"]
    o, g = both_protocols(w, inp, head, label="markov resident V=%d B=%d" % (V, B))
    g2, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    gs, _ = gpu_draft(markov_head(w, 8, dca.EXEC_STEPWISE), inp.H, inp.L_base, inp.last_tok)
    for k in ("tokens", "L_final", "u"):
        assert np.array_equal(g[k], g2[k]), k
        assert np.array_equal(g[k], gs[k]), k


@pytest.mark.parametrize("mode", [dca.EXEC_AUTO, dca.EXEC_STEPWISE])
@pytest.mark.parametrize("V,B", [(20011, 40), (7001, 130), (7001, 256)])
def test_markov_batched_matrix_cores_match_oracle(V, B, mode):
    """B > 8: A_H and W2 on the matrix cores, in the batched persistent launch (each
    block forms its share of u from the table and counts itself in the position's
    arrival counter) or in the step launches (where teacher forcing takes the one W2
    launch over all B*K (row, position) pairs)."""
    sh = ds.HeadShape(d=512, h=256, r=256, V=V, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 64), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 65), sigma=0.5, peak="none")
    head = markov_head(w, B, mode)
    info = head.exec_info(B)
    assert info["persistent"] == (mode == dca.EXEC_AUTO) and info["w2_resident"] == info["persistent"]
    both_protocols(w, inp, head, label="markov batched V=%d B=%d mode=%d" % (V, B, mode))


def test_markov_position_batched_equals_per_position():
    """With a teacher the position-batched step launches equal the resident kernel's
    per-position draft bit for bit."""
    sh = ds.HeadShape(d=256, h=128, r=256, V=9001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 66), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 67), sigma=0.5, peak="none")
    y = ds.uniform_tokens((9, 68), (3, 16), sh.V)
    a, _ = gpu_draft(markov_head(w, 3), inp.H, inp.L_base, inp.last_tok, teacher=y)
    b, _ = gpu_draft(markov_head(w, 3, dca.EXEC_POSITION_BATCHED), inp.H, inp.L_base, inp.last_tok, teacher=y)
    for k in ("tokens", "L_final", "u"):
        assert np.array_equal(a[k], b[k]), k
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y, markov=True)
    check_teacher_forced(o, a)


@pytest.mark.parametrize("mode", [dca.EXEC_AUTO, dca.EXEC_STEPWISE])
def test_markov_out_of_range_tokens_flag_rows(mode):
    sh = ds.HeadShape(d=256, h=128, r=256, V=3001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 69), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 70), sigma=0.5, peak="none")
    last = inp.last_tok.copy()
    last[1] = sh.V  # out of range
    g, flags = gpu_draft(markov_head(w, 3, mode), inp.H, inp.L_base, last)
    assert flags == dca.FLAG_BAD_TOKEN
    assert (g["tokens"][1] == -1).all()
    o = oracle.draft(w, inp.H[[0, 2]], inp.L_base[[0, 2]], last[[0, 2]], markov=True)
    check_free_running(o, {k: v[[0, 2]] for k, v in g.items()})


def test_markov_rejects_state_arguments():
    sh = ds.HeadShape(d=64, h=32, r=256, V=1001, K=4, wdtype="bf16")
    w = ds.make_weights(sh, (9, 71))
    inp = ds.make_inputs(sh, 1, (9, 72), sigma=0.5, peak="none")
    head = markov_head(w, 1)
    S0 = dca.device_tensor(np.zeros((1, sh.h), np.float32))
    with pytest.raises(dca.DominoError):
        head.draft(dca.device_tensor(inp.H), dca.device_tensor(inp.L_base), dca.device_tensor(inp.last_tok),
                   S_init=S0)


@pytest.fixture(scope="module")
def w8b():
    log("generating Qwen3-8B-shaped head weights")
    return ds.make_weights(ds.QWEN3_8B, ds.WORKLOADS["qwen3_8b_b1"].weight_key)


@pytest.mark.slow
def test_markov_qwen3_8b_b1_full(w8b):
    """The Markov head at the 8B shape, B = 1 (the benchmark's --markov launch)."""
    wl = ds.WORKLOADS["qwen3_8b_b1"]
    inp = ds.make_inputs(wl.shape, 1, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    head = markov_head(w8b, 1)
    assert head.exec_info(1)["w2_resident"]
    both_protocols(w8b, inp, head, label="markov 8B B=1")
    y = ds.uniform_tokens((3, 5), (1, 16), wl.shape.V)
    o = oracle.draft(w8b, inp.H, inp.L_base, inp.last_tok, teacher=y, markov=True)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert flags == 0
    check_teacher_forced(o, g)


@pytest.mark.slow
def test_markov_qwen3_8b_b32_sampled_rows(w8b):
    """The Markov head at the 8B shape, B = 32 (the batched persistent launch); the
    oracle checks sampled rows."""
    wl = ds.WORKLOADS["qwen3_8b_b32"]
    rows = [0, 17, 31]
    inp = ds.make_inputs(wl.shape, wl.B, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    g, flags = gpu_draft(markov_head(w8b, wl.B), inp.H, inp.L_base, inp.last_tok, rows=rows)
    assert flags == 0
    sub = ds.make_inputs(wl.shape, rows, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    o = oracle.draft(w8b, sub.H, sub.L_base, sub.last_tok, markov=True)
    div = check_free_running(o, g)
    log("markov 8B B=32 sampled rows %s: diverged=%d" % (rows, div))


@pytest.mark.parametrize("B,mode", [(1, dca.EXEC_AUTO), (3, dca.EXEC_PERSISTENT | dca.EXEC_PLAIN_LAUNCH),
                                    (12, dca.EXEC_AUTO)])
def test_markov_bf16_lbase_and_plain_launch_equal_float32(B, mode):
    """bf16 base logits are widened exactly on the Markov paths too (resident kernel and
    matrix-core step launches), and a plain launch equals the cooperative one: the
    outputs equal a float32, cooperative call on the widened values bit for bit."""
    sh = ds.HeadShape(d=256, h=128, r=256, V=9001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 73), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 74), sigma=0.5, peak="none")
    L16 = ds.round_to_bf16_bits(inp.L_base)
    a, fa = gpu_draft(markov_head(w, B, mode, lbase_bf16=True), inp.H, L16, inp.last_tok)
    b, fb = gpu_draft(markov_head(w, B), inp.H, ds.bf16_bits_to_f32(L16), inp.last_tok)
    assert fa == 0 and fb == 0
    for k in ("tokens", "L_final", "u"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("B,mode", [(3, dca.EXEC_PERSISTENT | dca.EXEC_PLAIN_LAUNCH),
                                    (40, dca.EXEC_PERSISTENT | dca.EXEC_PLAIN_LAUNCH), (40, dca.EXEC_STEPWISE)])
def test_markov_hip_graph_replay_matches_eager(B, mode):
    """A Markov draft captured in a HIP graph and replayed three times, with eager drafts
    of other inputs on the same handle in between, equals the eager result bitwise."""
    sh = ds.HeadShape(d=256, h=64, r=256, V=7001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 75), gru_sensitive=True)
    head = markov_head(w, B, mode)
    inp = ds.make_inputs(sh, B, (9, 76), sigma=0.5, peak="none")
    other = ds.make_inputs(sh, B, (9, 77), sigma=0.5, peak="none")
    ref, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    H, L, lt = dca.device_tensor(inp.H), dca.device_tensor(inp.L_base), dca.device_tensor(inp.last_tok)
    Ho, Lo, lto = dca.device_tensor(other.H), dca.device_tensor(other.L_base), dca.device_tensor(other.last_tok)
    dev = H.device
    gout = {"tokens": torch.empty((B, 16), dtype=torch.int32, device=dev),
            "L_final": torch.empty((B, 16, sh.V), dtype=torch.float32, device=dev),
            "u": torch.empty((B, 16, sh.r), dtype=torch.float32, device=dev)}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            head.draft(H, L, lt, want_logits=True, want_state=True, out=gout)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        head.draft(H, L, lt, want_logits=True, want_state=True, out=gout)
    for rep in range(3):
        for k in gout:
            gout[k].fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        for k in ("tokens", "L_final", "u"):
            assert np.array_equal(gout[k].cpu().numpy(), ref[k]), "replay %d: %s" % (rep, k)
        eager = head.draft(Ho, Lo, lto, want_logits=True)
        torch.cuda.synchronize()
        assert eager["tokens"].shape == (B, 16)
    assert head.check_error() == 0
