"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

Inputs come from the seeded generator; expected values come from the oracle
on the same inputs.  Protocols and tolerances are in gpu_common.py.
"""
import os

import numpy as np
import pytest
import torch

import causal_draft_correction_amd as dca
import domino_synth as ds
import oracle
from gpu_common import (GAP_TOL, compare_free_running, compare_teacher_forced, gpu_draft, log, make_head)

pytestmark = pytest.mark.gpu

MODES = [("persistent", dca.EXEC_PERSISTENT), ("stepwise", dca.EXEC_STEPWISE)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dca.load_library()


def run_both_protocols(w, inp, head, S_init=None, lf_tol=2e-2, s_tol=1e-4, u_tol=1e-4, label=""):
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, S_init=S_init)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, S_init=S_init)
    assert flags == 0
    div = compare_free_running(o, g, lf_tol, s_tol, u_tol)
    # teacher forcing with the oracle's own draft isolates per-step error
    ot = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=o["tokens"], S_init=S_init)
    gt, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=o["tokens"], S_init=S_init)
    assert flags == 0
    compare_teacher_forced(ot, gt, lf_tol, s_tol, u_tol)
    log("%s: free-running rows diverged=%d, L_final err fr=%.3g tf=%.3g, S err tf=%.3g" % (
        label, div, np.abs(o["L_final"][:, :1] - g["L_final"][:, :1]).max(),
        np.abs(ot["L_final"] - gt["L_final"]).max(), np.abs(ot["S"] - gt["S"]).max()))
    return o, g


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("mode_name,mode", MODES)
def test_tiny_fp32_head(mode_name, mode, fold):
    w, inp = ds.make_workload("tiny")
    head = make_head(w, 1, mode, fold=fold)
    run_both_protocols(w, inp, head, lf_tol=1e-4, label="tiny/%s/fold=%d" % (mode_name, fold))
    S0 = np.random.default_rng(0).standard_normal((1, w.shape.h)).astype(np.float32)
    run_both_protocols(w, inp, head, S_init=S0, lf_tol=1e-4, label="tiny+S_init/%s/fold=%d" % (mode_name, fold))


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("mode_name,mode", MODES)
@pytest.mark.parametrize("K", [16, 5, 1])
def test_ragged_bf16_gru_sensitive(mode_name, mode, K, fold):
    """V, d, h chosen so no tile or block partition divides them; GRU-sensitive
    weights and no planted peak so that the fed-back tokens change the logits."""
    sh = ds.HeadShape(d=520, h=136, r=64, V=5003, K=K, wdtype="bf16")
    w = ds.make_weights(sh, (9, 40), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 41), sigma=0.5, peak="none")
    head = make_head(w, 4, mode, fold=fold)
    run_both_protocols(w, inp, head, label="ragged K=%d/%s/fold=%d" % (K, mode_name, fold))


@pytest.mark.parametrize("fold", [False, True])
def test_random_teacher_and_state_init(fold):
    sh = ds.HeadShape(d=256, h=128, r=32, V=3001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 42), gru_sensitive=True)
    inp = ds.make_inputs(sh, 2, (9, 43), sigma=0.5, peak="none")
    y = ds.uniform_tokens((9, 44), (2, 16), sh.V)
    S0 = np.random.default_rng(1).standard_normal((2, sh.h)).astype(np.float32)
    for mode in (dca.EXEC_PERSISTENT, dca.EXEC_STEPWISE):
        head = make_head(w, 2, mode, fold=fold)
        o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y, S_init=S0)
        g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y, S_init=S0)
        assert flags == 0
        compare_teacher_forced(o, g)


@pytest.mark.parametrize("fold", [False, True])
def test_persistent_and_stepwise_are_bitwise_equal_and_deterministic(fold):
    sh = ds.HeadShape(d=520, h=136, r=64, V=5003, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 45), gru_sensitive=True)
    inp = ds.make_inputs(sh, 4, (9, 46), sigma=0.5, peak="none")
    a, _ = gpu_draft(make_head(w, 4, dca.EXEC_PERSISTENT, fold=fold), inp.H, inp.L_base, inp.last_tok)
    hp = make_head(w, 4, dca.EXEC_PERSISTENT, fold=fold)
    b, _ = gpu_draft(hp, inp.H, inp.L_base, inp.last_tok)
    b2, _ = gpu_draft(hp, inp.H, inp.L_base, inp.last_tok)
    c, _ = gpu_draft(make_head(w, 4, dca.EXEC_STEPWISE, fold=fold), inp.H, inp.L_base, inp.last_tok)
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(b[k], b2[k]), k
        assert np.array_equal(a[k], c[k]), k


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("mode", [dca.EXEC_PERSISTENT, dca.EXEC_STEPWISE])
def test_batch_rows_are_independent(mode, fold):
    sh = ds.HeadShape(d=256, h=64, r=32, V=2000, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 47), gru_sensitive=True)
    inp = ds.make_inputs(sh, 5, (9, 48), sigma=0.5, peak="none")
    head = make_head(w, 5, mode, fold=fold)
    full, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    for b in (0, 3):
        one, _ = gpu_draft(head, inp.H[b:b + 1], inp.L_base[b:b + 1], inp.last_tok[b:b + 1])
        for k in ("tokens", "L_final", "S", "u"):
            assert np.array_equal(one[k][0], full[k][b]), (b, k)


@pytest.mark.parametrize("mode", [dca.EXEC_PERSISTENT, dca.EXEC_STEPWISE])
def test_zero_W2_ties_nan_signed_zero(mode):
    """W2 = 0: L_final must equal L_base bitwise and tokens follow numpy.argmax
    (first index among equal maxima, first NaN wins, -0 == +0)."""
    sh = ds.HeadShape(d=64, h=32, r=16, V=777, K=16, wdtype="f32")
    w = ds.make_weights(sh, (9, 49))
    w.W2 = np.zeros_like(w.W2)
    inp = ds.make_inputs(sh, 3, (9, 50), sigma=2.0, peak="none")
    L = inp.L_base.copy()
    L[0, 1, 300] = L[0, 1, 30] = 100.0
    L[0, 2, :] = -1.0
    L[0, 2, 500] = -0.0
    L[0, 2, 400] = 0.0
    L[1, 3, 600] = np.nan
    L[1, 3, 700] = np.nan
    L[1, 3, 2] = np.inf
    L[2, 0, :] = 5.0
    L[2, 5, 776] = 50.0  # last index
    g, flags = gpu_draft(make_head(w, 3, mode), inp.H, L, inp.last_tok)
    assert flags == 0
    assert np.array_equal(g["L_final"].view(np.uint32), L.view(np.uint32)) or np.array_equal(
        np.nan_to_num(g["L_final"], nan=1e30), np.nan_to_num(L, nan=1e30))
    assert np.array_equal(g["tokens"], np.argmax(L, axis=-1))
    assert g["tokens"][0, 1] == 30 and g["tokens"][0, 2] == 400 and g["tokens"][1, 3] == 600
    assert g["tokens"][2, 0] == 0 and g["tokens"][2, 5] == 776


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("mode", [dca.EXEC_PERSISTENT, dca.EXEC_STEPWISE])
def test_out_of_range_tokens_flag_rows(mode, fold):
    sh = ds.HeadShape(d=64, h=32, r=16, V=500, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 51), gru_sensitive=True)
    inp = ds.make_inputs(sh, 4, (9, 52), sigma=0.5, peak="none")
    last = inp.last_tok.copy()
    last[1] = sh.V
    head = make_head(w, 4, mode, fold=fold)
    g, flags = gpu_draft(head, inp.H, inp.L_base, last)
    assert flags & dca.FLAG_BAD_TOKEN
    assert np.all(g["tokens"][1] == -1)
    o = oracle.draft(w, inp.H, inp.L_base, last)
    assert list(o["flags"]) == [0, 1, 0, 0]
    good = [0, 2, 3]
    compare_free_running(o, {k: v[good] for k, v in g.items()}, orows=good)
    # a bad teacher id in a used position; the last teacher entry is never read
    y = ds.uniform_tokens((9, 53), (4, 16), sh.V)
    y[2, 4] = -7
    y[3, 15] = 10 ** 6
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert flags & dca.FLAG_BAD_TOKEN
    assert np.all(g["tokens"][2] == -1) and np.all(g["tokens"][3] >= 0)
    # flags were cleared by the read
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    assert flags == 0


def test_barrier_timeout_is_reported_not_hung(monkeypatch):
    """A spin limit of 0 (read from the environment at create) forces every
    waiting block out of its first barrier: the launch must end and report
    DOMINO_FLAG_SYNC_TIMEOUT; a second head created afterwards with the default
    limit must work normally."""
    sh = ds.HeadShape(d=64, h=32, r=16, V=500, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 54))
    inp = ds.make_inputs(sh, 1, (9, 55))
    monkeypatch.setenv("DOMINO_BARRIER_SPIN_LIMIT", "0")
    head = make_head(w, 1, dca.EXEC_PERSISTENT)
    monkeypatch.delenv("DOMINO_BARRIER_SPIN_LIMIT")
    _, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    assert flags & dca.FLAG_SYNC_TIMEOUT
    head2 = make_head(w, 1, dca.EXEC_PERSISTENT)
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    g, flags = gpu_draft(head2, inp.H, inp.L_base, inp.last_tok)
    assert flags == 0
    compare_free_running(o, g)


@pytest.mark.parametrize("B,wd,r,fold", [(1, "bf16", 16, False), (1, "bf16", 256, False), (3, "f32", 32, False),
                                         (40, "bf16", 256, True)])
def test_same_handle_recovers_after_a_timeout(B, wd, r, fold):
    """The spin limit set to 0 on a live handle makes a draft time out (the
    streaming, the resident B = 1 and the batched B = 40 persistent kernels);
    after check_error and the default limit restored, the same handle (same
    workspace, barrier generations restarted) drafts correctly again, twice."""
    sh = ds.HeadShape(d=128, h=64, r=r, V=700, K=16, wdtype=wd)
    w = ds.make_weights(sh, (9, 58, r))
    inp = ds.make_inputs(sh, B, (9, 59, r))
    head = make_head(w, B, dca.EXEC_PERSISTENT, fold=fold)
    assert head.exec_info(B)["persistent"]
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    assert flags == 0
    head.set_spin_limit(0)
    _, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    assert flags & dca.FLAG_SYNC_TIMEOUT
    head.set_spin_limit(1 << 22)
    for _ in range(2):
        g2, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
        assert flags == 0
        compare_free_running(o, g2)
        assert np.array_equal(g2["tokens"], g["tokens"])


def test_output_tensors_are_checked_before_any_launch():
    """Caller-supplied out tensors of the wrong shape, dtype, layout or device are
    refused on the host; nothing is written."""
    sh = ds.HeadShape(d=64, h=32, r=16, V=500, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 56))
    head = make_head(w, 2, dca.EXEC_AUTO)
    inp = ds.make_inputs(sh, 2, (9, 57))
    H, L, lt = dca.device_tensor(inp.H), dca.device_tensor(inp.L_base), dca.device_tensor(inp.last_tok)
    dev = "cuda"
    bad = [{"tokens": torch.empty((2, 15), dtype=torch.int32, device=dev)},
           {"tokens": torch.empty((2, 16), dtype=torch.int64, device=dev)},
           {"tokens": torch.empty((16, 2), dtype=torch.int32, device=dev).t()},
           {"tokens": torch.empty((2, 16), dtype=torch.int32)},
           {"L_final": torch.empty((2, 16, 499), dtype=torch.float32, device=dev)},
           {"S": torch.empty((2, 16, 32), dtype=torch.bfloat16, device=dev)},
           {"u": torch.empty((1, 16, 16), dtype=torch.float32, device=dev)},
           {"logits": torch.empty((2, 16, 500), dtype=torch.float32, device=dev)}]
    for o in bad:
        with pytest.raises(ValueError):
            head.draft(H, L, lt, out=o)
    good = {"tokens": torch.full((2, 16), -7, dtype=torch.int32, device=dev),
            "u": torch.empty((2, 16, 16), dtype=torch.float32, device=dev)}
    g = head.draft(H, L, lt, out=good)
    torch.cuda.synchronize()
    assert g["tokens"] is good["tokens"] and int(good["tokens"].min()) >= 0


def test_host_validation_of_draft_arguments():
    sh = ds.HeadShape(d=64, h=32, r=16, V=500, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 56))
    head = make_head(w, 2, dca.EXEC_AUTO)
    inp = ds.make_inputs(sh, 3, (9, 57))
    with pytest.raises(dca.DominoError) as e:
        gpu_draft(head, inp.H, inp.L_base, inp.last_tok)  # B = 3 > max_batch = 2
    assert e.value.code == -1


# ------------------------------------------------------------------ full sizes
@pytest.fixture(scope="module")
def w8b():
    log("generating Qwen3-8B-shaped head weights")
    return ds.make_weights(ds.QWEN3_8B, ds.WORKLOADS["qwen3_8b_b1"].weight_key)


@pytest.mark.slow
@pytest.mark.parametrize("fold", [False, True])
def test_qwen3_4b_b1_full(fold):
    w, inp = ds.make_workload("qwen3_4b_b1")
    head = make_head(w, 1, fold=fold)
    run_both_protocols(w, inp, head, label="4B B=1 fold=%d" % fold)


@pytest.mark.slow
def test_qwen3_8b_b1_full(w8b):
    wl = ds.WORKLOADS["qwen3_8b_b1"]
    inp = ds.make_inputs(wl.shape, 1, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    for mode, fold in ((dca.EXEC_AUTO, True), (dca.EXEC_AUTO, False), (dca.EXEC_STEPWISE, False)):
        head = make_head(w8b, 1, mode, fold=fold)
        run_both_protocols(w8b, inp, head, label="8B B=1 mode=%d fold=%d" % (mode, fold))
        del head
    # a uniform random teacher as well
    y = ds.uniform_tokens((3, 2), (1, 16), wl.shape.V)
    o = oracle.draft(w8b, inp.H, inp.L_base, inp.last_tok, teacher=y)
    g, flags = gpu_draft(make_head(w8b, 1, fold=True), inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert flags == 0
    compare_teacher_forced(o, g)


@pytest.mark.slow
@pytest.mark.parametrize("name,rows,mode", [("qwen3_8b_b32", [0, 13, 31], dca.EXEC_AUTO),
                                            ("qwen3_8b_b256", [0, 101, 255], dca.EXEC_AUTO),
                                            ("qwen3_8b_b256", [0, 77, 255], dca.EXEC_STEPWISE)])
def test_qwen3_8b_batched_sampled_rows(w8b, name, rows, mode):
    """Full batch on the device (AUTO: the launch the benchmark times, the batched
    persistent kernel; and the step launches at B = 256), folded table, float32 L_base;
    the oracle checks sampled rows free running and teacher forced with its own draft."""
    wl = ds.WORKLOADS[name]
    inp = ds.make_inputs(wl.shape, wl.B, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    head = make_head(w8b, wl.B, mode, fold=True)
    assert head.exec_info(wl.B)["persistent"] == (mode == dca.EXEC_AUTO)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, rows=rows)
    assert flags == 0
    sub = ds.make_inputs(wl.shape, rows, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    o = oracle.draft(w8b, sub.H, sub.L_base, sub.last_tok)
    div = compare_free_running(o, g)
    log("%s sampled rows %s: diverged=%d" % (name, rows, div))
    y = np.zeros((wl.B, wl.shape.K), np.int32)
    y[rows] = o["tokens"]
    gt, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y, rows=rows)
    assert flags == 0
    compare_teacher_forced(o, gt)
    # accept length on synthetic verifier tokens built from the oracle draft
    tgt, k = ds.geometric_prefix_targets(o["tokens"], (4, 3), wl.shape.V)
    got = dca.accept_len(dca.device_tensor(g["tokens"]), dca.device_tensor(tgt)).cpu().numpy()
    assert np.array_equal(got, oracle.accept_len(g["tokens"], tgt))


@pytest.mark.slow
@pytest.mark.parametrize("name,rows,variant", [("qwen3_8b_b32", [0, 19, 31], "teacher"),
                                               ("qwen3_8b_b256", [0, 128, 255], "lbase_bf16")])
def test_qwen3_8b_batched_variants_sampled_rows(w8b, name, rows, variant):
    """The launches the benchmark times with --teacher and with --lbase-bf16 (the batched
    persistent kernel, folded table), at full size; the oracle checks sampled rows."""
    wl = ds.WORKLOADS[name]
    sh = wl.shape
    inp = ds.make_inputs(sh, wl.B, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    sub = ds.make_inputs(sh, rows, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    if variant == "teacher":
        y = ds.uniform_tokens(list(wl.row_key) + [9], (wl.B, sh.K), sh.V)
        g, flags = gpu_draft(make_head(w8b, wl.B, fold=True), inp.H, inp.L_base, inp.last_tok, teacher=y, rows=rows)
        assert flags == 0
        o = oracle.draft(w8b, sub.H, sub.L_base, sub.last_tok, teacher=y[rows])
        compare_teacher_forced(o, g)
    else:
        L16 = ds.round_to_bf16_bits(inp.L_base)
        g, flags = gpu_draft(make_head(w8b, wl.B, fold=True, lbase_bf16=True), inp.H, L16, inp.last_tok, rows=rows)
        assert flags == 0
        o = oracle.draft(w8b, sub.H, ds.bf16_bits_to_f32(L16[rows]), sub.last_tok)
        div = compare_free_running(o, g)
        log("%s bf16 L_base sampled rows %s: diverged=%d" % (name, rows, div))


# ------------------------------------------------------------------ accept length
@pytest.mark.parametrize("B,K", [(1, 16), (37, 16), (256, 16), (1000, 16), (300, 5), (7, 1)])
def test_accept_len_bit_exact(B, K):
    rng = np.random.default_rng(B * 31 + K)
    draft = rng.integers(0, 151936, size=(B, K)).astype(np.int32)
    tgt, k = ds.geometric_prefix_targets(draft, (8, B, K), 151936)
    tgt[0] = draft[0]  # a full match (k = K)
    if B > 1:
        tgt[1, 0] = draft[1, 0] + 1  # k = 0
    got = dca.accept_len(dca.device_tensor(draft), dca.device_tensor(tgt)).cpu().numpy()
    ref = oracle.accept_len(draft, tgt)
    assert np.array_equal(got, ref)
    assert got[0] == K


# ------------------------------------------------------------------ resident W2 (bf16, r = 256)
@pytest.mark.parametrize("V,B,fold", [(5003, 1, True), (5003, 3, False), (5003, 8, True), (160000, 2, True),
                                      (160000, 6, False)])
def test_resident_w2_slice_matches_oracle(V, B, fold):
    """r = 256 bf16 heads keep each block's W2 slice on chip and multiply it on the
    matrix cores (u split into bf16 hi + lo parts).  V = 160000 (625 rows per block
    on 256 compute units) puts tiles beyond the register share into LDS; B = 6 uses
    batch rows 4..5 of the packed epilogue.  Compared with the oracle, with the
    streaming launch and run to run."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=V, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 60), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 61), sigma=0.5, peak="none")
    head = make_head(w, B, dca.EXEC_PERSISTENT, fold=fold)
    info = head.exec_info(B)
    assert info["persistent"] and info["w2_resident"] and info["grid"] > 0, info
    run_both_protocols(w, inp, head, label="resident V=%d B=%d fold=%d" % (V, B, fold))
    a, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    b, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], b[k]), k
    pl = make_head(w, B, dca.EXEC_PERSISTENT | dca.EXEC_PLAIN_LAUNCH, fold=fold)
    d, _ = gpu_draft(pl, inp.H, inp.L_base, inp.last_tok)
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], d[k]), "plain launch " + k
    st = make_head(w, B, dca.EXEC_PERSISTENT | dca.EXEC_STREAM_W2, fold=fold)
    assert st.exec_info(B)["w2_resident"] is False
    assert make_head(w, B, dca.EXEC_STEPWISE, fold=fold).exec_info(B) == {"persistent": False, "w2_resident": False,
                                                                          "grid": 0}
    c, _ = gpu_draft(st, inp.H, inp.L_base, inp.last_tok)
    assert np.abs(c["L_final"] - a["L_final"]).max() < 1e-4


# ------------------------------------------------------------------ batched W2 on the matrix cores (r = 256)
@pytest.mark.parametrize("V,B,fold", [(20011, 9, True), (20011, 40, False), (7001, 130, True), (7001, 128, True),
                                      (20011, 256, False)])
def test_batched_w2_matrix_cores_match_oracle(V, B, fold):
    """Stepwise launches of bf16 r = 256 heads run W2 as a matrix-core GEMM (u as bf16
    hi + lo operand rows, fused L_base add and argmax); above 8 rows the state-phase
    dot products also run on the matrix cores (S as bf16 hi + lo).  B = 40 leaves a
    partial 32-row group, B = 130 a second 128-row batch tile with two rows."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=V, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 70), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 71), sigma=0.5, peak="none")
    head = make_head(w, B, dca.EXEC_STEPWISE, fold=fold)
    assert head.exec_info(B) == {"persistent": False, "w2_resident": False, "grid": 0}
    run_both_protocols(w, inp, head, label="batched W2 V=%d B=%d fold=%d" % (V, B, fold))
    a, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    b, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("B", [40, 128])
def test_batched_w2_zero_correction_ties_nan_signed_zero(B):
    """Matrix-core W2 launches (B = 128: W2 streamed into registers; B = 40: staged
    through LDS) with W2 = 0: L_final equals L_base (up to the sign of zero) and the
    tokens follow numpy.argmax: the first of equal maxima, the first NaN, -0 == +0, and
    index 0 for a row of -inf, with specials placed across vocabulary ranges."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=7001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 74))
    w.W2 = np.zeros_like(w.W2)
    inp = ds.make_inputs(sh, B, (9, 75), sigma=2.0, peak="none")
    L = inp.L_base.copy()
    L[0, 1, [5, 6999]] = 100.0       # tie across the first and last vocabulary ranges
    L[1, 2, :] = -1.0
    L[1, 2, [3000, 77]] = [-0.0, 0.0]  # -0 == +0: the lower index wins
    L[2, 3, [4000, 900]] = np.nan      # first NaN wins
    L[2, 3, 10] = np.inf
    L[B - 1, 4, :] = -np.inf           # all -inf: index 0
    L[B - 1, 5, 6000] = np.inf
    head = make_head(w, B, dca.EXEC_STEPWISE, fold=True)
    g, flags = gpu_draft(head, inp.H, L, inp.last_tok)
    assert flags == 0
    np.testing.assert_array_equal(g["tokens"], np.argmax(L, axis=-1))
    assert g["tokens"][0, 1] == 5 and g["tokens"][1, 2] == 77 and g["tokens"][2, 3] == 900
    assert g["tokens"][B - 1, 4] == 0 and g["tokens"][B - 1, 5] == 6000
    assert np.array_equal(np.nan_to_num(g["L_final"], nan=1e30), np.nan_to_num(L, nan=1e30))


@pytest.mark.parametrize("B", [1, 4])
def test_batched_w2_equals_resident_kernel_bitwise(B):
    """Both matrix-core W2 paths form each logit as L_base + (hi + lo) from the same
    instruction on the same operands, and share the state phase arithmetic (at
    B = 1 the resident launch forms A_H inside each block, in phase_ah's order):
    the stepwise launches and the resident persistent launch agree bitwise."""
    sh = ds.HeadShape(d=5136, h=64, r=256, V=9001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 72), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 73), sigma=0.5, peak="none")
    pers = make_head(w, 4, dca.EXEC_PERSISTENT, fold=True)
    assert pers.exec_info(B)["w2_resident"]
    a, _ = gpu_draft(pers, inp.H, inp.L_base, inp.last_tok)
    c, _ = gpu_draft(make_head(w, 4, dca.EXEC_STEPWISE, fold=True), inp.H, inp.L_base, inp.last_tok)
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], c[k]), k


def test_resident_handle_with_varying_batch():
    """One handle drafting many blocks with few rows and then one with more rows.
    The exchange words of rows a launch does not draft are left from earlier
    launches; they must never pass for current ones, however many launches lie
    between (the 16-bit u tags and the 14-bit argmax generations wrap).  4095
    single-row blocks bring the barrier generation past 2^16 before the
    three-row block, which must equal the same block drafted on a fresh handle."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=9001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 80), gru_sensitive=True)
    inp3 = ds.make_inputs(sh, 3, (9, 81), sigma=0.5, peak="none")
    inp1 = ds.make_inputs(sh, 1, (9, 82), sigma=0.5, peak="none")
    head = make_head(w, 4, dca.EXEC_PERSISTENT, fold=True)
    assert head.exec_info(1)["w2_resident"] and head.exec_info(3)["w2_resident"]
    H1, L1 = dca.device_tensor(inp1.H), dca.device_tensor(inp1.L_base)
    t1 = dca.device_tensor(np.asarray(inp1.last_tok, np.int32))
    out = {"tokens": torch.empty((1, sh.K), dtype=torch.int32, device=H1.device)}
    for i in range(4095):
        head.draft(H1, L1, t1, out=out)
        if i % 1024 == 0:
            log("single-row draft %d" % i)
    torch.cuda.synchronize()
    assert head.check_error() == 0
    one, _ = gpu_draft(make_head(w, 1, dca.EXEC_PERSISTENT, fold=True), inp1.H, inp1.L_base, inp1.last_tok,
                       want_logits=False, want_state=False)
    assert np.array_equal(out["tokens"].cpu().numpy(), one["tokens"])
    a, flags = gpu_draft(head, inp3.H, inp3.L_base, inp3.last_tok)
    assert flags == 0
    b, _ = gpu_draft(make_head(w, 4, dca.EXEC_PERSISTENT, fold=True), inp3.H, inp3.L_base, inp3.last_tok)
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], b[k]), k
    o = oracle.draft(w, inp3.H, inp3.L_base, inp3.last_tok)
    compare_free_running(o, a)


@pytest.mark.parametrize("wd,V,B", [("bf16", 9001, 3), ("f32", 3001, 2), ("bf16", 9001, 8)])
def test_position_batched_teacher_forcing_equals_per_position(wd, V, B):
    """With a teacher the step launches run the GRU chain first and then one W2
    launch over all B*K (row, position) pairs.  The products are the same
    instructions on the same operands as per position, so the result equals the
    persistent (per-position) launch bit for bit: matrix-core W2 for the bf16
    r = 256 head (at B = 8 the 128 rows take the kernel that streams W2 into
    registers), the VALU W2 kernel for the fp32 head."""
    sh = ds.HeadShape(d=1040 if wd == "bf16" else 136, h=64, r=256 if wd == "bf16" else 32, V=V, K=16, wdtype=wd)
    w = ds.make_weights(sh, (9, 90), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 91), sigma=0.5, peak="none")
    y = ds.uniform_tokens((9, 92), (B, 16), V)
    mb = max(B, 4)
    a, fa = gpu_draft(make_head(w, mb, dca.EXEC_PERSISTENT, fold=True), inp.H, inp.L_base, inp.last_tok, teacher=y)
    pb = make_head(w, mb, dca.EXEC_POSITION_BATCHED, fold=True)
    assert pb.exec_info(B)["persistent"]  # exec_info reports the launch without a teacher
    c, fc = gpu_draft(pb, inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert fa == 0 and fc == 0
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], c[k]), k
    # without u_out the u of every position goes through the workspace
    d, _ = gpu_draft(pb, inp.H, inp.L_base, inp.last_tok, teacher=y, want_state=False)
    assert np.array_equal(d["tokens"], a["tokens"]) and np.array_equal(d["L_final"], a["L_final"])


@pytest.mark.parametrize("mode", [dca.EXEC_POSITION_BATCHED, dca.EXEC_AUTO])
def test_position_batched_teacher_forcing_matches_oracle_at_larger_batch(mode):
    """B = 40 with a teacher (position-batched: matrix-core launches over 640 rows;
    auto: the batched resident launch), against the oracle's teacher-forced draft;
    one row has an invalid teacher id."""
    sh = ds.HeadShape(d=256, h=64, r=256, V=7001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 93), gru_sensitive=True)
    B = 40
    inp = ds.make_inputs(sh, B, (9, 94), sigma=0.5, peak="none")
    y = ds.uniform_tokens((9, 95), (B, 16), sh.V)
    y[7, 3] = sh.V + 5
    head = make_head(w, B, mode, fold=True)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert flags == dca.FLAG_BAD_TOKEN
    assert (g["tokens"][7] == -1).all()
    good = [b for b in range(B) if b != 7]
    o = oracle.draft(w, inp.H[good], inp.L_base[good], inp.last_tok[good], teacher=y[good])
    sub = {k: v[good] for k, v in g.items()}
    compare_teacher_forced(o, sub)


BF16_LBASE_CASES = {
    # name: (wdtype, d, h, r, V, B, max_batch, exec mode, fold, teacher)
    "resident_b1": ("bf16", 1040, 64, 256, 5003, 1, 4, dca.EXEC_PERSISTENT, True, False),
    "resident_b3": ("bf16", 1040, 64, 256, 5003, 3, 4, dca.EXEC_PERSISTENT, True, False),
    "resident_lds_tiles": ("bf16", 256, 64, 256, 160000, 2, 2, dca.EXEC_PERSISTENT, True, False),
    "resident_unfolded": ("bf16", 256, 64, 256, 5003, 1, 1, dca.EXEC_PERSISTENT, False, False),
    "streamed_w2": ("bf16", 256, 64, 256, 5003, 2, 2, dca.EXEC_PERSISTENT | dca.EXEC_STREAM_W2, True, False),
    "batched_resident": ("bf16", 256, 64, 256, 20011, 40, 40, dca.EXEC_AUTO, True, False),
    "batched_matrix_cores": ("bf16", 256, 64, 256, 20011, 40, 40, dca.EXEC_STEPWISE, True, False),
    "batched_resident_teacher": ("bf16", 256, 64, 256, 7001, 9, 9, dca.EXEC_AUTO, True, True),
    "position_batched": ("bf16", 256, 64, 256, 7001, 9, 9, dca.EXEC_POSITION_BATCHED, True, True),
    "position_batched_b8": ("bf16", 256, 64, 256, 7001, 8, 8, dca.EXEC_POSITION_BATCHED, True, True),
    "batched_b128": ("bf16", 256, 64, 256, 7001, 128, 128, dca.EXEC_STEPWISE, True, False),
    "batched_resident_b128": ("bf16", 256, 64, 256, 7008, 128, 128, dca.EXEC_AUTO, True, False),
    "f32_stepwise": ("f32", 136, 64, 32, 3001, 3, 4, dca.EXEC_STEPWISE, False, False),
    "f32_persistent": ("f32", 136, 64, 32, 3001, 3, 4, dca.EXEC_PERSISTENT, True, False),
}


@pytest.mark.parametrize("case", sorted(BF16_LBASE_CASES))
def test_bf16_lbase_equals_float32_of_the_same_values(case):
    """With DOMINO_LBASE_BF16 every path widens each base logit exactly, so a call
    with bf16 L_base equals a float32 call on the widened values bit for bit."""
    wd, d, h, r, V, B, mb, mode, fold, tf = BF16_LBASE_CASES[case]
    sh = ds.HeadShape(d=d, h=h, r=r, V=V, K=16, wdtype=wd)
    w = ds.make_weights(sh, (9, 100), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 101), sigma=0.5, peak="none")
    L16 = ds.round_to_bf16_bits(inp.L_base)
    L32 = ds.bf16_bits_to_f32(L16)
    y = ds.uniform_tokens((9, 102), (B, 16), V) if tf else None
    a, fa = gpu_draft(make_head(w, mb, mode, fold=fold, lbase_bf16=True), inp.H, L16, inp.last_tok, teacher=y)
    b, fb = gpu_draft(make_head(w, mb, mode, fold=fold), inp.H, L32, inp.last_tok, teacher=y)
    assert fa == 0 and fb == 0
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], b[k]), k


def test_bf16_lbase_resident_matches_oracle():
    sh = ds.HeadShape(d=256, h=64, r=256, V=5003, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 103), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 104), sigma=0.5, peak="none")
    L16 = ds.round_to_bf16_bits(inp.L_base)
    inp32 = ds.BlockInputs(inp.H, ds.bf16_bits_to_f32(L16), inp.last_tok, inp.temperature, inp.peak_ids)
    head = make_head(w, 3, dca.EXEC_PERSISTENT, fold=True, lbase_bf16=True)
    o = oracle.draft(w, inp32.H, inp32.L_base, inp32.last_tok)
    g, flags = gpu_draft(head, inp.H, L16, inp.last_tok)
    assert flags == 0
    compare_free_running(o, g)


@pytest.mark.parametrize("B", [64, 70])
def test_lds_staged_state_dots_match_oracle(B):
    """h = 256 and B >= 64 take the LDS-staged state launch: a ragged batch tile
    (B = 70) and a ragged weight tile (r + 3h = 800 rows), against the oracle in
    both protocols."""
    sh = ds.HeadShape(d=256, h=256, r=32, V=3001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 110), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (9, 111), sigma=0.5, peak="none")
    head = make_head(w, B, dca.EXEC_AUTO, fold=True)
    assert not head.exec_info(B)["persistent"]
    run_both_protocols(w, inp, head, label="staged state dots B=%d" % B)


@pytest.mark.parametrize("case", ["step_launches_b40", "resident_plain_launch_b3", "batched_resident_plain_launch_b40"])
def test_hip_graph_replay_matches_eager(case):
    """A draft call captured in a HIP graph (no memset nodes: the library clears with
    kernels) replayed several times, with eager draft calls of other inputs on the same
    handle in between; every replay equals the eager result bitwise."""
    sh = ds.HeadShape(d=256, h=64, r=256, V=7001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 120), gru_sensitive=True)
    if case == "step_launches_b40":
        B, mode = 40, dca.EXEC_STEPWISE
    elif case == "batched_resident_plain_launch_b40":
        B, mode = 40, dca.EXEC_PLAIN_LAUNCH
    else:
        B, mode = 3, dca.EXEC_PERSISTENT | dca.EXEC_PLAIN_LAUNCH
    head = make_head(w, B, mode, fold=True)
    inp = ds.make_inputs(sh, B, (9, 121), sigma=0.5, peak="none")
    other = ds.make_inputs(sh, B, (9, 122), sigma=0.5, peak="none")
    ref, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    H, L, lt = dca.device_tensor(inp.H), dca.device_tensor(inp.L_base), dca.device_tensor(inp.last_tok)
    Ho, Lo, lto = dca.device_tensor(other.H), dca.device_tensor(other.L_base), dca.device_tensor(other.last_tok)
    dev = H.device
    gout = {"tokens": torch.empty((B, 16), dtype=torch.int32, device=dev),
            "L_final": torch.empty((B, 16, sh.V), dtype=torch.float32, device=dev),
            "S": torch.empty((B, 16, sh.h), dtype=torch.float32, device=dev),
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
        for k in ("tokens", "L_final", "S", "u"):
            assert np.array_equal(gout[k].cpu().numpy(), ref[k]), "replay %d: %s" % (rep, k)
        eager = head.draft(Ho, Lo, lto, want_logits=True)  # other work on the same handle in between
        torch.cuda.synchronize()
        assert eager["tokens"].shape == (B, 16)
    assert head.check_error() == 0


def test_side_streams_and_two_handles_concurrently():
    """Calls are ordered on the caller's stream: a draft on a side stream equals the
    default-stream result, and two handles drafting on two streams at once (step
    launches) each equal their own sequential result."""
    sh = ds.HeadShape(d=256, h=64, r=256, V=7001, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (9, 130), gru_sensitive=True)
    B = 24
    ia = ds.make_inputs(sh, B, (9, 131), sigma=0.5, peak="none")
    ib = ds.make_inputs(sh, B, (9, 132), sigma=0.5, peak="none")
    ha, hb = make_head(w, B, dca.EXEC_STEPWISE, fold=True), make_head(w, B, dca.EXEC_STEPWISE, fold=True)
    ra, _ = gpu_draft(ha, ia.H, ia.L_base, ia.last_tok)
    rb, _ = gpu_draft(hb, ib.H, ib.L_base, ib.last_tok)
    dev = [dca.device_tensor(x) for x in (ia.H, ia.L_base, ia.last_tok, ib.H, ib.L_base, ib.last_tok)]
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        with torch.cuda.stream(sa):
            oa = ha.draft(dev[0], dev[1], dev[2], want_logits=True, want_state=True)
        with torch.cuda.stream(sb):
            ob = hb.draft(dev[3], dev[4], dev[5], want_logits=True, want_state=True)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        for k in ("tokens", "L_final", "S", "u"):
            assert np.array_equal(oa[k].cpu().numpy(), ra[k]), k
            assert np.array_equal(ob[k].cpu().numpy(), rb[k]), k
    assert ha.check_error() == 0 and hb.check_error() == 0
