"""GPU parity of the batched resident-W2 persistent launch (9 <= B <= 256 rows,
bf16 weights, r = 256, folded gate table): each block keeps its W2 slice in
registers for the whole block draft, and the GRU update and state dot products
are distributed over the grid between barriers.  Compared with the fp64 oracle
in both protocols (tolerances in gpu_common.py), and bitwise with itself where
the arithmetic is the same (bf16 L_base widened, plain launch, row subsets,
repeated runs).
"""
import numpy as np
import pytest
import torch

import causal_draft_correction_amd as dca
import domino_synth as ds
import oracle
from gpu_common import compare_free_running, compare_teacher_forced, gpu_draft, log, make_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dca.load_library()


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def batched_head(w, max_batch, mode=dca.EXEC_PERSISTENT, lbase_bf16=False):
    head = make_head(w, max_batch, mode, fold=True, lbase_bf16=lbase_bf16)
    return head


def both_protocols(w, inp, head, S_init=None, label=""):
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, S_init=S_init)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, S_init=S_init)
    assert flags == 0
    div = compare_free_running(o, g)
    ot = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=o["tokens"], S_init=S_init)
    gt, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=o["tokens"], S_init=S_init)
    assert flags == 0
    compare_teacher_forced(ot, gt)
    log("%s: diverged rows %d, L_final err tf %.3g, S err tf %.3g, u err tf %.3g" % (
        label, div, np.abs(ot["L_final"] - gt["L_final"]).max(), np.abs(ot["S"] - gt["S"]).max(),
        np.abs(ot["u"] - gt["u"]).max()))
    return o, g


def test_exec_info_reports_the_batched_resident_launch():
    sh = ds.HeadShape(d=256, h=64, r=256, V=20000, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 1))
    head = batched_head(w, 300)
    for B in (9, 40, 256):
        assert head.exec_info(B) == {"persistent": True, "w2_resident": True, "grid": cus()}, B
    # past B = 256 a forced persistent launch is refused
    with pytest.raises(RuntimeError):
        head.exec_info(257)
    # AUTO takes the batched launch for 8 < B <= 256 and the step launches above
    auto = batched_head(w, 300, dca.EXEC_AUTO)
    for B in (9, 40, 48, 49, 256):
        assert auto.exec_info(B) == {"persistent": True, "w2_resident": True, "grid": cus()}, B
    assert auto.exec_info(8)["w2_resident"] and auto.exec_info(8)["persistent"]
    assert auto.exec_info(257) == {"persistent": False, "w2_resident": False, "grid": 0}
    assert make_head(w, 40, fold=False).exec_info(40)["persistent"] is False
    assert make_head(w, 40, dca.EXEC_STEPWISE, fold=True).exec_info(40)["persistent"] is False
    # a forced persistent launch at B > 8 takes the batched kernel
    assert make_head(w, 40, dca.EXEC_PERSISTENT, fold=True).exec_info(40)["grid"] == cus()


# (V, B, h): V % 4 == 0 copies L_base rows in 16-byte pieces, other V value by value;
# B = 9 and 17 leave ragged batch groups, 130 a ragged last 16-row group, 256 the
# largest batch; h = 64, 128 and 256 run one, two and four 64-wide stages of the state dots
CASES = [(20000, 9, 64), (20011, 40, 64), (7001, 130, 128), (4096, 256, 64), (9000, 17, 256), (5003, 64, 64)]


@pytest.mark.parametrize("V,B,h", CASES)
def test_batched_resident_matches_oracle(V, B, h):
    sh = ds.HeadShape(d=256, h=h, r=256, V=V, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 2, V, B), gru_sensitive=True)
    inp = ds.make_inputs(sh, B, (12, 3, V, B), sigma=0.5, peak="none")
    head = batched_head(w, B)
    assert head.exec_info(B)["grid"] == cus()
    both_protocols(w, inp, head, label="batched resident V=%d B=%d h=%d" % (V, B, h))


def test_batched_resident_state_init_and_random_teacher():
    sh = ds.HeadShape(d=256, h=128, r=256, V=12000, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 4), gru_sensitive=True)
    B = 40
    inp = ds.make_inputs(sh, B, (12, 5), sigma=0.5, peak="none")
    S_init = np.random.default_rng(12).normal(0, 0.5, size=(B, sh.h)).astype(np.float32)
    head = batched_head(w, B)
    both_protocols(w, inp, head, S_init=S_init, label="batched resident S_init")
    y = ds.uniform_tokens((12, 6), (B, 16), sh.V)
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y, S_init=S_init)
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y, S_init=S_init)
    assert flags == 0
    compare_teacher_forced(o, g)


@pytest.mark.parametrize("V,B", [(7001, 40), (8000, 130)])
def test_batched_resident_zero_correction_ties_nan_signed_zero(V, B):
    """W2 = 0: L_final equals L_base (up to the sign of zero) and the tokens follow
    numpy.argmax (the first of equal maxima, the first NaN, -0 == +0, index 0 for a
    row of -inf), with the specials in different blocks' vocabulary ranges."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=V, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 7))
    w.W2 = np.zeros_like(w.W2)
    inp = ds.make_inputs(sh, B, (12, 8), sigma=2.0, peak="none")
    L = inp.L_base.copy()
    L[0, 1, [5, V - 2]] = 100.0
    L[1, 2, :] = -1.0
    L[1, 2, [3000, 77]] = [-0.0, 0.0]
    L[2, 3, [4000, 900]] = np.nan
    L[2, 3, 10] = np.inf
    L[B - 1, 4, :] = -np.inf
    L[B - 1, 5, V - 1] = np.inf
    L[17, 6, [V - 1, 0]] = 50.0
    head = batched_head(w, B)
    g, flags = gpu_draft(head, inp.H, L, inp.last_tok)
    assert flags == 0
    np.testing.assert_array_equal(g["tokens"], np.argmax(L, axis=-1))
    assert g["tokens"][0, 1] == 5 and g["tokens"][1, 2] == 77 and g["tokens"][2, 3] == 900
    assert g["tokens"][B - 1, 4] == 0 and g["tokens"][B - 1, 5] == V - 1 and g["tokens"][17, 6] == 0
    assert np.array_equal(np.nan_to_num(g["L_final"], nan=1e30), np.nan_to_num(L, nan=1e30))


def test_batched_resident_out_of_range_tokens_flag_rows():
    sh = ds.HeadShape(d=256, h=64, r=256, V=6000, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 9), gru_sensitive=True)
    B = 24
    inp = ds.make_inputs(sh, B, (12, 10), sigma=0.5, peak="none")
    lt = inp.last_tok.copy()
    lt[3] = sh.V
    lt[11] = -2
    head = batched_head(w, B)
    g, flags = gpu_draft(head, inp.H, inp.L_base, lt)
    assert flags == dca.FLAG_BAD_TOKEN
    assert (g["tokens"][3] == -1).all() and (g["tokens"][11] == -1).all()
    good = [b for b in range(B) if b not in (3, 11)]
    o = oracle.draft(w, inp.H[good], inp.L_base[good], lt[good])
    compare_free_running(o, {k: v[good] for k, v in g.items()})
    y = ds.uniform_tokens((12, 11), (B, 16), sh.V)
    y[5, 14] = sh.V + 3
    y[6, 15] = sh.V + 3  # the last teacher entry is never read
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert flags == dca.FLAG_BAD_TOKEN
    assert (g["tokens"][5] == -1).all() and (g["tokens"][6] != -1).all()


def test_batched_resident_deterministic_rows_independent_and_plain_launch():
    """Run to run bitwise; a row's results do not depend on the other rows of the
    call (the first 20 rows alone give the same bits); the plain launch equals the
    cooperative one."""
    sh = ds.HeadShape(d=256, h=128, r=256, V=11000, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 12), gru_sensitive=True)
    B = 40
    inp = ds.make_inputs(sh, B, (12, 13), sigma=0.5, peak="none")
    head = batched_head(w, B)
    a, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    b, _ = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    c, _ = gpu_draft(head, inp.H[:20], inp.L_base[:20], inp.last_tok[:20])
    d, fd = gpu_draft(batched_head(w, B, dca.EXEC_PLAIN_LAUNCH), inp.H, inp.L_base, inp.last_tok)
    assert fd == 0
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k][:20], c[k]), k
        assert np.array_equal(a[k], d[k]), k


def test_batched_resident_store_logits_and_bf16_lbase():
    """Launches without the L_final store and with bf16 base logits (widened exactly)
    give the same tokens, states and activations bit for bit; with V % 8 != 0 and
    V % 8 == 0 (value-by-value and 16-byte L_base copies)."""
    for V in (9001, 9008):
        sh = ds.HeadShape(d=256, h=64, r=256, V=V, K=16, wdtype="bf16")
        w = ds.make_weights(sh, (12, 14, V), gru_sensitive=True)
        B = 33
        inp = ds.make_inputs(sh, B, (12, 15, V), sigma=0.5, peak="none")
        L16 = ds.round_to_bf16_bits(inp.L_base)
        L32 = ds.bf16_bits_to_f32(L16)
        a, fa = gpu_draft(batched_head(w, B, lbase_bf16=True), inp.H, L16, inp.last_tok)
        b, fb = gpu_draft(batched_head(w, B), inp.H, L32, inp.last_tok)
        c, fc = gpu_draft(batched_head(w, B), inp.H, L32, inp.last_tok, want_logits=False)
        assert fa == fb == fc == 0
        for k in ("tokens", "L_final", "S", "u"):
            assert np.array_equal(a[k], b[k]), (V, k)
        for k in ("tokens", "S", "u"):
            assert np.array_equal(b[k], c[k]), (V, k)
        o = oracle.draft(w, inp.H, L32, inp.last_tok)
        compare_free_running(o, a)


def test_batched_resident_handle_with_varying_batch():
    """The argmax words carry 14-bit generation tags.  520 drafts of 9 rows (32
    generations each: past 2^14) leave the words of rows 9..63 from the last launch
    that wrote them; a 64-row draft afterwards must equal the same draft on a fresh
    handle."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=4096, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 16), gru_sensitive=True)
    i64 = ds.make_inputs(sh, 64, (12, 17), sigma=0.5, peak="none")
    i9 = ds.make_inputs(sh, 9, (12, 18), sigma=0.5, peak="none")
    head = batched_head(w, 64)
    a0, _ = gpu_draft(head, i64.H, i64.L_base, i64.last_tok)
    H9, L9, t9 = dca.device_tensor(i9.H), dca.device_tensor(i9.L_base), dca.device_tensor(i9.last_tok)
    out = {"tokens": torch.empty((9, 16), dtype=torch.int32, device=H9.device)}
    for i in range(520):
        head.draft(H9, L9, t9, out=out)
        if i % 128 == 0:
            log("9-row draft %d" % i)
    torch.cuda.synchronize()
    assert head.check_error() == 0
    one, _ = gpu_draft(batched_head(w, 9), i9.H, i9.L_base, i9.last_tok, want_logits=False, want_state=False)
    assert np.array_equal(out["tokens"].cpu().numpy(), one["tokens"])
    # without a check_error in between (which restarts the generations), 520 more, then 64 rows
    for i in range(520):
        head.draft(H9, L9, t9, out=out)
    a, flags = gpu_draft(head, i64.H, i64.L_base, i64.last_tok)
    assert flags == 0
    for k in ("tokens", "L_final", "S", "u"):
        assert np.array_equal(a[k], a0[k]), k


def test_batched_resident_timeout_is_reported_not_hung(monkeypatch):
    """A spin limit of 0 forces the blocks out of their first wait: the launch ends and
    reports DOMINO_FLAG_SYNC_TIMEOUT; a head created afterwards (default spin limit)
    drafts correctly."""
    sh = ds.HeadShape(d=128, h=64, r=256, V=5000, K=16, wdtype="bf16")
    w = ds.make_weights(sh, (12, 19), gru_sensitive=True)
    B = 20
    inp = ds.make_inputs(sh, B, (12, 20), sigma=0.5, peak="none")
    monkeypatch.setenv("DOMINO_BARRIER_SPIN_LIMIT", "0")
    head = batched_head(w, B)
    monkeypatch.delenv("DOMINO_BARRIER_SPIN_LIMIT")
    _, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok)
    assert flags & dca.FLAG_SYNC_TIMEOUT
    ref, flags = gpu_draft(batched_head(w, B), inp.H, inp.L_base, inp.last_tok)
    assert flags == 0
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    compare_free_running(o, ref)


@pytest.mark.slow
@pytest.mark.parametrize("name,rows", [("qwen3_8b_b32", [0, 13, 31]), ("qwen3_8b_b256", [0, 101, 255])])
def test_qwen3_8b_batched_resident_sampled_rows(name, rows):
    """The launch the benchmark times (folded table, batched resident kernel) at full
    size; the oracle checks sampled rows free running and teacher forced with its own
    draft."""
    wl = ds.WORKLOADS[name]
    sh = wl.shape
    w = ds.make_weights(sh, wl.weight_key)
    inp = ds.make_inputs(sh, wl.B, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    sub = ds.make_inputs(sh, rows, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    head = batched_head(w, wl.B)
    assert head.exec_info(wl.B)["grid"] == cus()
    g, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, rows=rows)
    assert flags == 0
    o = oracle.draft(w, sub.H, sub.L_base, sub.last_tok)
    div = compare_free_running(o, g)
    y = np.zeros((wl.B, sh.K), np.int32)
    y[rows] = o["tokens"]
    gt, flags = gpu_draft(head, inp.H, inp.L_base, inp.last_tok, teacher=y, rows=rows)
    assert flags == 0
    compare_teacher_forced(o, gt)
    log("%s batched resident sampled rows %s: diverged=%d" % (name, rows, div))
