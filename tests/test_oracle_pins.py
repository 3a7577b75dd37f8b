"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the pin and the passage (page + section) it follows.  The
pages are: the paper.oopus.info review ("review"), the news.sig.ai article
("article"), the researchpapers.dev summary ("summary") and the Hugging Face
papers mirror ("HF page").  All tests here run on the CPU.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import domino_synth as ds
import oracle
from oracle import numpy_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_shape(V=37, d=24, h=16, r=8, K=16, wdtype="f32"):
    return ds.HeadShape(d=d, h=h, r=r, V=V, K=K, wdtype=wdtype)


def weights_f64(w, name):
    a = getattr(w, name)
    if w.shape.wdtype == "f32":
        return a.astype(np.float64)
    return ds.bf16_bits_to_f32(a).astype(np.float64)


def zero_like(a):
    return np.zeros_like(a)


def silu64(x):
    return torch.nn.functional.silu(torch.from_numpy(x)).numpy()


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_P1_zero_W2_gives_base_argmax(wdtype):
    """W2 = 0 removes the correction (review, section 二: L_final = L_base + W2 sigma(...)):
    L_final equals L_base exactly and the greedy draft (article, 'Domino怎么做') is
    numpy.argmax of L_base, including its first-occurrence rule for exact ties and NaN."""
    sh = small_shape(V=50, wdtype=wdtype)
    w = ds.make_weights(sh, (9, 1))
    w.W2 = zero_like(w.W2)
    inp = ds.make_inputs(sh, 3, (9, 2), sigma=2.0, peak="none")
    L = inp.L_base.copy()
    # planted specials: exact tie between two maxima, a -0/+0 tie at the top, and NaNs
    L[0, 1, 7] = L[0, 1, 30] = 100.0
    L[0, 2, :] = -1.0
    L[0, 2, 11] = -0.0
    L[0, 2, 4] = 0.0
    L[1, 3, 20] = np.nan
    L[1, 3, 40] = np.nan
    L[1, 3, 2] = np.inf
    L[2, 0, :] = 5.0  # all equal
    o = oracle.draft(w, inp.H, L, inp.last_tok)
    np.testing.assert_array_equal(o["L_final"], L.astype(np.float64))
    np.testing.assert_array_equal(o["tokens"], np.argmax(L, axis=-1))
    assert o["tokens"][0, 1] == 7 and o["tokens"][0, 2] == 4 and o["tokens"][1, 3] == 20
    assert o["tokens"][2, 0] == 0


# ---------------------------------------------------------------- P2
def test_P2_zero_gru_reduces_to_position_wise_head():
    """Zero GRU parameters with S_init = 0 keep S at 0, so the head is the
    position-wise map L_base + W2 SiLU(W1[:, :d] H_i) (review, section 二 formula) and
    the draft no longer depends on the fed-back tokens: free running equals teacher
    forcing for any teacher (review, section 二, Teacher Forcing)."""
    sh = small_shape(V=61, d=32, h=16, r=8)
    w = ds.make_weights(sh, (9, 3))
    for k in ("W_ih", "W_hh", "b_ih", "b_hh"):
        setattr(w, k, zero_like(getattr(w, k)))
    inp = ds.make_inputs(sh, 2, (9, 4), sigma=0.5, peak="none")
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    assert np.all(o["S"] == 0.0)
    W1 = weights_f64(w, "W1")
    W2 = weights_f64(w, "W2")
    H = inp.H.astype(np.float64)
    ref = inp.L_base.astype(np.float64) + silu64(H @ W1[:, :sh.d].T) @ W2.T
    np.testing.assert_allclose(o["L_final"], ref, rtol=0, atol=1e-12)
    y = ds.uniform_tokens((9, 5), (2, sh.K), sh.V)
    ot = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y)
    np.testing.assert_array_equal(ot["L_final"], o["L_final"])
    np.testing.assert_array_equal(ot["tokens"], o["tokens"])


# ---------------------------------------------------------------- P3
def test_P3_all_zero_gru_halves_state():
    """All GRU parameters zero: r = z = sigmoid(0) = 1/2, n = tanh(0) = 0, so every
    GRUCell step maps s to s/2; with the anchor step S_k = 0.5^(k+1) S_init exactly."""
    sh = small_shape(V=29, d=16, h=24, r=8)
    w = ds.make_weights(sh, (9, 6))
    for k in ("W_ih", "W_hh", "b_ih", "b_hh"):
        setattr(w, k, zero_like(getattr(w, k)))
    inp = ds.make_inputs(sh, 1, (9, 7), peak="uniform")
    S0 = np.random.default_rng(5).standard_normal((1, sh.h)).astype(np.float32)
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, S_init=S0)
    for k in range(sh.K):
        np.testing.assert_array_equal(o["S"][0, k], 0.5 ** (k + 1) * S0[0].astype(np.float64))


# ---------------------------------------------------------------- P4
def test_P4_bias_only_gru_closed_form():
    """W_ih = W_hh = 0 with non-zero biases: gates are constants
    r* = sig(b_ir + b_hr), z* = sig(b_iz + b_hz), n* = tanh(b_in + r* b_hn), and the
    PyTorch GRUCell recursion s' = (1 - z*) n* + z* s has the closed form
    S_k = n* + z*^(k+1) (S_init - n*).  A swapped gate order or the other
    placement of the reset gate (r* applied before the b_hn bias) fails this."""
    sh = small_shape(V=23, d=16, h=32, r=8)
    w = ds.make_weights(sh, (9, 8))
    w.W_ih = zero_like(w.W_ih)
    w.W_hh = zero_like(w.W_hh)
    rng = np.random.default_rng(11)
    w.b_ih = rng.standard_normal(3 * sh.h).astype(np.float32)
    w.b_hh = rng.standard_normal(3 * sh.h).astype(np.float32)
    inp = ds.make_inputs(sh, 1, (9, 9), peak="uniform")
    S0 = rng.standard_normal((1, sh.h)).astype(np.float32)
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, S_init=S0)
    h = sh.h
    bi = w.b_ih.astype(np.float64)
    bh = w.b_hh.astype(np.float64)
    rs = 1 / (1 + np.exp(-(bi[:h] + bh[:h])))
    zs = 1 / (1 + np.exp(-(bi[h:2 * h] + bh[h:2 * h])))
    ns = np.tanh(bi[2 * h:] + rs * bh[2 * h:])
    for k in range(sh.K):
        ref = ns + zs ** (k + 1) * (S0[0].astype(np.float64) - ns)
        np.testing.assert_allclose(o["S"][0, k], ref, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P5
@pytest.mark.parametrize("wdtype,teacher", [("f32", False), ("bf16", False), ("f32", True)])
def test_P5_state_chain_matches_torch_grucell(wdtype, teacher):
    """Random weights, GRU-sensitive scale: the oracle's S_0..S_{K-1} equal a chain of
    torch.nn.GRUCell (float64) fed E[last_tok], then E of each draft token (review,
    section 二: the GRU reads the draft embeddings of preceding positions) or of the
    teacher token (review, Teacher Forcing); and its corrections equal
    W2 SiLU(W1 [H_i; S_{i-1}]) evaluated with torch.nn.functional.linear/silu."""
    sh = small_shape(V=41, d=24, h=16, r=8, wdtype=wdtype)
    w = ds.make_weights(sh, (9, 10), gru_sensitive=True)
    inp = ds.make_inputs(sh, 2, (9, 11), sigma=0.3, peak="none")
    rng = np.random.default_rng(3)
    S0 = (0.5 * rng.standard_normal((2, sh.h))).astype(np.float32)
    y = ds.uniform_tokens((9, 12), (2, sh.K), sh.V) if teacher else None
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y, S_init=S0)
    cell = torch.nn.GRUCell(sh.d, sh.h, bias=True, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(weights_f64(w, "W_ih")))
        cell.weight_hh.copy_(torch.from_numpy(weights_f64(w, "W_hh")))
        cell.bias_ih.copy_(torch.from_numpy(weights_f64(w, "b_ih")))
        cell.bias_hh.copy_(torch.from_numpy(weights_f64(w, "b_hh")))
    E = torch.from_numpy(weights_f64(w, "E"))
    W1 = torch.from_numpy(weights_f64(w, "W1"))
    W2 = torch.from_numpy(weights_f64(w, "W2"))
    H = inp.H.astype(np.float64) if wdtype == "f32" else ds.bf16_bits_to_f32(inp.H).astype(np.float64)
    for b in range(2):
        with torch.no_grad():
            s = cell(E[int(inp.last_tok[b])][None], torch.from_numpy(S0[b].astype(np.float64))[None])[0]
            for i in range(sh.K):
                np.testing.assert_allclose(o["S"][b, i], s.numpy(), rtol=0, atol=1e-12)
                cat = torch.cat([torch.from_numpy(H[b, i]), s])
                corr = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(cat, W1)), W2)
                np.testing.assert_allclose(o["L_final"][b, i] - inp.L_base[b, i], corr.numpy(), rtol=0, atol=1e-12)
                if i + 1 < sh.K:
                    tok = int(y[b, i]) if teacher else int(o["tokens"][b, i])
                    s = cell(E[tok][None], s[None])[0]


# ---------------------------------------------------------------- P6
def test_P6_teacher_equal_to_draft_reproduces_it():
    """Teacher forcing with the free-running draft as the teacher feeds the GRU the
    same tokens, so tokens and logits are bitwise identical."""
    sh = small_shape(V=45, d=24, h=16, r=8)
    w = ds.make_weights(sh, (9, 13), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 14), sigma=0.3, peak="none")
    fr = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    tf = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=fr["tokens"])
    np.testing.assert_array_equal(tf["tokens"], fr["tokens"])
    np.testing.assert_array_equal(tf["L_final"], fr["L_final"])
    np.testing.assert_array_equal(tf["S"], fr["S"])


# ---------------------------------------------------------------- P7
def test_P7_brute_force_fixed_point_is_the_greedy_draft():
    """Tiny vocabulary: over every teacher sequence y_1..y_{K-1} in V^(K-1), exactly
    one is a fixed point of teacher forcing (its own greedy outputs), and it equals
    the free-running greedy draft.  A shifted or mis-wired feedback index breaks
    either uniqueness or the equality."""
    sh = small_shape(V=5, d=8, h=8, r=4, K=5)
    w = ds.make_weights(sh, (9, 15), gru_sensitive=True)
    # make the state matter: scale W1's state columns further
    w.W1[:, sh.d:] *= 4.0
    inp = ds.make_inputs(sh, 1, (9, 16), sigma=0.2, peak="none")
    fr = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)["tokens"][0]
    fixed = []
    seqs = np.array(list(itertools.product(range(sh.V), repeat=sh.K - 1)), dtype=np.int32)
    teach = np.concatenate([seqs, np.zeros((len(seqs), 1), np.int32)], axis=1)
    n = len(seqs)
    out = oracle.draft(w, np.repeat(inp.H, n, 0), np.repeat(inp.L_base, n, 0), np.repeat(inp.last_tok, n),
                       teacher=teach, want_logits=False, want_state=False, threads=1)["tokens"]
    for j in range(n):
        if np.array_equal(out[j, :sh.K - 1], seqs[j]):
            fixed.append(j)
    assert len(fixed) == 1
    np.testing.assert_array_equal(out[fixed[0]], fr)
    # the draft must actually depend on the fed tokens, or the test pins nothing
    assert len({tuple(x) for x in out}) > 1


# ---------------------------------------------------------------- P8
def test_P8_parameter_count_matches_page():
    """The review (section 二) says the Domino head adds about 56 million parameters;
    with h = 1024 and r = 256 (same section) at the Qwen3-8B-shaped width d = 4096 and
    vocabulary 151936, W1 + W2 + GRU matrices give 55,934,976 (55,941,120 with GRU
    biases), within 1% of that figure."""
    facts = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
    sh = ds.QWEN3_8B
    assert sh.h == facts["gru_hidden"]["value"] and sh.r == facts["rank"]["value"]
    assert sh.K == facts["block_size"]["value"]
    n = oracle.param_count(sh.d, sh.h, sh.r, sh.V)
    nb = oracle.param_count(sh.d, sh.h, sh.r, sh.V, with_bias=True)
    assert n == 256 * (4096 + 1024) + 151936 * 256 + 3 * 1024 * 4096 + 3 * 1024 * 1024 == 55_934_976
    assert nb - n == 6 * 1024
    target = facts["head_params_approx"]["value"]
    assert abs(n - target) / target < facts["head_params_approx"]["rel_tol"]
    assert abs(nb - target) / target < facts["head_params_approx"]["rel_tol"]


# ---------------------------------------------------------------- P9
def test_P9_correction_does_not_depend_on_base_logits():
    """The correction is added in logit space (review, section 二); under teacher
    forcing the GRU inputs are fixed, so L_final - L_base must not change when L_base
    is redrawn."""
    sh = small_shape(V=53, d=24, h=16, r=8)
    w = ds.make_weights(sh, (9, 17), gru_sensitive=True)
    a = ds.make_inputs(sh, 2, (9, 18), sigma=1.0, peak="none")
    b = ds.make_inputs(sh, 2, (9, 19), sigma=1.0, peak="none")
    y = ds.uniform_tokens((9, 20), (2, sh.K), sh.V)
    oa = oracle.draft(w, a.H, a.L_base, a.last_tok, teacher=y)
    ob = oracle.draft(w, a.H, b.L_base, a.last_tok, teacher=y)
    np.testing.assert_allclose(oa["L_final"] - a.L_base, ob["L_final"] - b.L_base, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(oa["S"], ob["S"])


# ---------------------------------------------------------------- P10
def test_P10_vocab_permutation_equivariance():
    """Relabelling the vocabulary (rows of W2 and E, columns of L_base, the anchor
    token) relabels the draft and permutes the logits; a transposed W2 or E, or a
    gather by the wrong index, breaks it."""
    sh = small_shape(V=47, d=24, h=16, r=8)
    w = ds.make_weights(sh, (9, 21), gru_sensitive=True)
    inp = ds.make_inputs(sh, 2, (9, 22), sigma=0.5, peak="none")
    perm = np.random.default_rng(7).permutation(sh.V)  # old id v -> new id perm[v]
    inv = np.argsort(perm)
    wp = ds.HeadWeights(sh, w.W1, w.W2[inv], w.W_ih, w.W_hh, w.b_ih, w.b_hh, w.E[inv])
    Lp = inp.L_base[:, :, inv]
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    op = oracle.draft(wp, inp.H, Lp, perm[inp.last_tok].astype(np.int32))
    np.testing.assert_array_equal(op["tokens"], perm[o["tokens"]])
    np.testing.assert_array_equal(op["L_final"], o["L_final"][:, :, inv])


# ---------------------------------------------------------------- P11
def test_P11_rows_are_independent():
    """Batch rows do not interact: a row run alone equals that row of a batch."""
    sh = small_shape(V=31, d=16, h=16, r=8)
    w = ds.make_weights(sh, (9, 23), gru_sensitive=True)
    inp = ds.make_inputs(sh, 4, (9, 24), sigma=0.5, peak="none")
    full = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    one = ds.make_inputs(sh, [2], (9, 24), sigma=0.5, peak="none")
    np.testing.assert_array_equal(one.L_base[0], inp.L_base[2])
    o2 = oracle.draft(w, one.H, one.L_base, one.last_tok)
    np.testing.assert_array_equal(o2["tokens"][0], full["tokens"][2])
    np.testing.assert_array_equal(o2["L_final"][0], full["L_final"][2])


# ---------------------------------------------------------------- P12
def test_P12_accept_length_prefix_rule():
    """The verifier accepts the longest draft prefix equal to its own tokens (review,
    section 一; summary, 关键结果).  Targets built with a known matched length k give
    accept length k; k = 0 and k = K are covered."""
    rng = np.random.default_rng(0)
    draft = rng.integers(0, 1000, size=(64, 16)).astype(np.int32)
    tgt, k = ds.geometric_prefix_targets(draft, (4, 3), 1000)
    np.testing.assert_array_equal(oracle.accept_len(draft, tgt), k)
    assert len(set(k.tolist())) > 4  # the construction covers many lengths
    # explicit edges
    t2 = draft.copy()
    t2[0, 0] += 1          # k = 0
    t2[1, 15] += 1         # k = 15
    t2[3, 7] += 1          # k = 7 (later equal entries do not count)
    got = oracle.accept_len(draft, t2)
    assert got[0] == 0 and got[1] == 15 and got[2] == 16 and got[3] == 7
    assert np.all(got[4:] == 16)
    # K other than 16, and B = 1
    assert oracle.accept_len(draft[:1, :5], draft[:1, :5])[0] == 5


# ---------------------------------------------------------------- misc
def test_invalid_tokens_mark_row():
    """An anchor or used teacher token outside [0, V) makes the row invalid: tokens
    -1 and flag 1.  The last teacher entry is never fed to the GRU, so it is not
    checked."""
    sh = small_shape(V=19, d=16, h=8, r=8)
    w = ds.make_weights(sh, (9, 25))
    inp = ds.make_inputs(sh, 3, (9, 26), peak="uniform")
    last = inp.last_tok.copy()
    last[1] = sh.V
    o = oracle.draft(w, inp.H, inp.L_base, last)
    assert list(o["flags"]) == [0, 1, 0] and np.all(o["tokens"][1] == -1)
    y = np.zeros((3, sh.K), np.int32)
    y[0, 3] = -2
    y[2, sh.K - 1] = 10_000
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y)
    assert list(o["flags"]) == [1, 0, 0]


def test_gap_is_top1_minus_top2():
    sh = small_shape(V=57, d=16, h=8, r=8)
    w = ds.make_weights(sh, (9, 27))
    inp = ds.make_inputs(sh, 2, (9, 28), peak="uniform")
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    s = np.sort(o["L_final"], axis=-1)
    np.testing.assert_allclose(o["gap"], s[..., -1] - s[..., -2], rtol=0, atol=0)


@pytest.mark.parametrize("cfg", ["tiny", "bf16mini"])
def test_c_oracle_matches_numpy_rewrite(cfg):
    if cfg == "tiny":
        w, inp = ds.make_workload("tiny")
        S0 = None
    else:
        sh = ds.HeadShape(d=64, h=32, r=16, V=301, K=16, wdtype="bf16")
        w = ds.make_weights(sh, (9, 29), gru_sensitive=True)
        inp = ds.make_inputs(sh, 2, (9, 30), sigma=0.5, peak="none")
        S0 = np.random.default_rng(1).standard_normal((2, sh.h)).astype(np.float32)
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, S_init=S0)
    n = numpy_ref.draft(w, inp.H, inp.L_base, inp.last_tok, S_init=S0)
    np.testing.assert_array_equal(o["tokens"], n["tokens"])
    np.testing.assert_allclose(o["L_final"], n["L_final"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o["S"], n["S"], rtol=0, atol=1e-12)


def test_thread_count_does_not_change_results():
    w, inp = ds.make_workload("tiny")
    a = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, threads=1)
    b = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, threads=7)
    for k in ("tokens", "L_final", "S", "u", "gap"):
        np.testing.assert_array_equal(a[k], b[k])


# ---- greedy verify step (review section 一; summary, 关键结果 and 常见问题) ----

def test_V1_verify_target_tokens_are_numpy_argmax():
    """The target's greedy token of each row equals numpy.argmax on the float32
    logits, including planted ties (lowest index), NaN (the first NaN), a row
    of +-0, a row of -inf and the last index."""
    g = np.random.default_rng(7)
    B, K, V = 3, 5, 29
    lg = (g.standard_normal((B, K + 1, V)) * 3).astype(np.float32)
    lg[0, 0, [4, 9, 20]] = 50.0                  # exact tie: 4 wins
    lg[0, 1, 11] = np.nan
    lg[0, 1, 3] = np.nan                         # first NaN: 3
    lg[0, 2] = 0.0
    lg[0, 2, :7] = -0.0                          # -0 == +0: index 0
    lg[1, 0] = -np.inf                           # all -inf: index 0
    lg[1, 1, V - 1] = 99.0                       # last index
    lg[2, 3, 0] = np.inf
    lg[2, 3, 5] = np.inf                         # +inf tie: 0
    draft = g.integers(0, V, size=(B, K)).astype(np.int32)
    r = oracle.verify(lg, draft)
    assert np.array_equal(r["target"], np.argmax(lg, axis=-1).astype(np.int32))


def test_V2_verify_accept_and_next_on_constructed_blocks():
    """Planted target tokens (generator construction, not the oracle): the accept
    length equals the constructed k (target equals the draft on the first k
    positions and differs at k), and the committed token is the planted token of
    row k -- the target's own choice after the accepted prefix."""
    vi = ds.make_verify_inputs(24, 16, 997, (21, 0))
    r = oracle.verify(vi.logits, vi.draft)
    assert np.array_equal(r["target"], vi.planted)
    assert np.array_equal(r["accept"], np.minimum(vi.k, 16))
    assert np.array_equal(r["next"], vi.planted[np.arange(24), vi.k])
    assert (vi.k == 16).any() and (vi.k == 0).any()  # both ends of the range occur
    # all drafts accepted: the committed token is the argmax of the extra row K
    full = oracle.verify(vi.logits, vi.planted[:, :16])
    assert np.array_equal(full["accept"], np.full(24, 16))
    assert np.array_equal(full["next"], vi.planted[:, 16])


def test_V3_speculative_loop_reproduces_greedy_decoding():
    """Lossless property stated by the pages (summary, 关键结果 and 常见问题:
    every accepted token is the target's own): with a toy greedy target whose
    logits depend on the last two tokens, drafting noisy guesses, verifying them
    and committing accept + the verify token reproduces plain greedy decoding
    token for token, whatever the guesses."""
    V, K, N = 11, 5, 60
    g = np.random.default_rng(3)
    table = g.standard_normal((V, V, V)).astype(np.float32)

    def logits_after(seq):
        return table[seq[-2], seq[-1]]

    ref = [1, 2]
    while len(ref) < 2 + N:
        ref.append(int(np.argmax(logits_after(ref))))
    for p_wrong in (0.0, 0.3, 1.0):
        seq = [1, 2]
        steps = 0
        while len(seq) < 2 + N:
            # guesses: the true continuation, each token corrupted with probability p_wrong
            guess, ctx = [], list(seq)
            for _ in range(K):
                t = int(np.argmax(logits_after(ctx)))
                if g.random() < p_wrong:
                    t = (t + 1 + int(g.integers(0, V - 1))) % V
                guess.append(t)
                ctx.append(t)
            rows = np.stack([logits_after(seq + guess[:j]) for j in range(K + 1)])[None]
            r = oracle.verify(rows, np.asarray([guess], np.int32))
            a = int(r["accept"][0])
            seq += guess[:a] + [int(r["next"][0])]
            steps += 1
        assert seq[:2 + N] == ref, "p_wrong=%g" % p_wrong
        if p_wrong == 0.0:
            assert steps == -(-N // (K + 1))  # every step commits K + 1 tokens


# ---------------------------------------------------------------- Markov head
# The article (section 从Domino看DSpark) names a Markov head, the default of
# DSpark, beside an RNN head that corresponds to Domino's causal encoder; it
# gives no formula.  Reading: each position is conditioned on the preceding
# token alone, S_i = GRU(E[x_i], 0) with x_0 = last_tok.

def gru_cell64(w):
    sh = w.shape
    cell = torch.nn.GRUCell(sh.d, sh.h, bias=True, dtype=torch.float64)
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(weights_f64(w, "W_ih")))
        cell.weight_hh.copy_(torch.from_numpy(weights_f64(w, "W_hh")))
        cell.bias_ih.copy_(torch.from_numpy(weights_f64(w, "b_ih")))
        cell.bias_hh.copy_(torch.from_numpy(weights_f64(w, "b_hh")))
    return cell


def test_M1_markov_equals_recurrent_when_no_state_is_carried():
    """With W_hh = 0 and the update gate shut (its W_ih rows zero, its input bias
    -1e4, so z = 0 exactly in double), the recurrent cell's new state n no longer
    depends on the old one: the recurrent head and the Markov head then give
    bitwise the same tokens, logits and states.  With the recurrence switched back
    on they differ, so the Markov flag really changes the state feed."""
    sh = small_shape(V=43, d=24, h=16, r=8)
    w = ds.make_weights(sh, (9, 40), gru_sensitive=True)
    inp = ds.make_inputs(sh, 3, (9, 41), sigma=0.3, peak="none")
    rec = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    mk = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, markov=True)
    assert np.abs(rec["S"][:, 1:] - mk["S"][:, 1:]).max() > 1e-3
    np.testing.assert_array_equal(rec["S"][:, 0], mk["S"][:, 0])  # anchor: both start from zero
    h = sh.h
    w.W_hh = zero_like(w.W_hh)
    w.W_ih[h:2 * h] = 0.0
    w.b_ih[h:2 * h] = -1e4
    w.b_hh[h:2 * h] = 0.0
    rec = oracle.draft(w, inp.H, inp.L_base, inp.last_tok)
    mk = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, markov=True)
    for k in ("tokens", "L_final", "S", "u"):
        np.testing.assert_array_equal(rec[k], mk[k])


@pytest.mark.parametrize("wdtype,teacher", [("f32", False), ("bf16", False), ("f32", True)])
def test_M2_markov_states_are_grucell_from_zero(wdtype, teacher):
    """Markov head: S_i equals torch.nn.GRUCell (float64) applied to E[x_i] with a
    zero hidden state, x_0 = last_tok and x_i the draft token (or teacher token) of
    position i - 1, and each correction equals W2 SiLU(W1 [H_i; S_i]) evaluated with
    torch.nn.functional (review, section 二 formula)."""
    sh = small_shape(V=41, d=24, h=16, r=8, wdtype=wdtype)
    w = ds.make_weights(sh, (9, 42), gru_sensitive=True)
    inp = ds.make_inputs(sh, 2, (9, 43), sigma=0.3, peak="none")
    y = ds.uniform_tokens((9, 44), (2, sh.K), sh.V) if teacher else None
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y, markov=True)
    cell = gru_cell64(w)
    E = torch.from_numpy(weights_f64(w, "E"))
    W1 = torch.from_numpy(weights_f64(w, "W1"))
    W2 = torch.from_numpy(weights_f64(w, "W2"))
    H = inp.H.astype(np.float64) if wdtype == "f32" else ds.bf16_bits_to_f32(inp.H).astype(np.float64)
    zero = torch.zeros(1, sh.h, dtype=torch.float64)
    for b in range(2):
        for i in range(sh.K):
            x = int(inp.last_tok[b]) if i == 0 else int(y[b, i - 1] if teacher else o["tokens"][b, i - 1])
            with torch.no_grad():
                s = cell(E[x][None], zero)[0]
                cat = torch.cat([torch.from_numpy(H[b, i]), s])
                corr = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(cat, W1)), W2)
            np.testing.assert_allclose(o["S"][b, i], s.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(o["L_final"][b, i] - inp.L_base[b, i], corr.numpy(), rtol=0, atol=1e-12)


def test_M3_markov_position_depends_only_on_the_preceding_token():
    """Teacher forced Markov head: changing the teacher token of position j changes
    the logits of position j + 1 and of no other position (bitwise); the recurrent
    head changes every later position."""
    sh = small_shape(V=47, d=24, h=16, r=8)
    w = ds.make_weights(sh, (9, 45), gru_sensitive=True)
    inp = ds.make_inputs(sh, 1, (9, 46), sigma=0.3, peak="none")
    y = ds.uniform_tokens((9, 47), (1, sh.K), sh.V)
    j = 5
    y2 = y.copy()
    y2[0, j] = (y[0, j] + 1) % sh.V
    a = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y, markov=True)["L_final"][0]
    b = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y2, markov=True)["L_final"][0]
    changed = [i for i in range(sh.K) if not np.array_equal(a[i], b[i])]
    assert changed == [j + 1]
    ra = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y)["L_final"][0]
    rb = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, teacher=y2)["L_final"][0]
    assert [i for i in range(sh.K) if not np.array_equal(ra[i], rb[i])] == list(range(j + 1, sh.K))


def test_M4_markov_low_rank_input_is_a_per_token_table():
    """Since S_i is a function of one token, W1 [H_i; S_i] = W1_H H_i + M[x_i] with a
    per-token table M[t] = W1_S GRU(E[t], 0) (V x r).  The oracle's u equals SiLU of
    that sum with M built for every token by torch (float64)."""
    sh = small_shape(V=29, d=24, h=16, r=8)
    w = ds.make_weights(sh, (9, 48), gru_sensitive=True)
    inp = ds.make_inputs(sh, 2, (9, 49), sigma=0.3, peak="none")
    o = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, markov=True)
    cell = gru_cell64(w)
    E = torch.from_numpy(weights_f64(w, "E"))
    W1 = weights_f64(w, "W1")
    with torch.no_grad():
        S_all = cell(E, torch.zeros(sh.V, sh.h, dtype=torch.float64)).numpy()
    M = S_all @ W1[:, sh.d:].T
    for b in range(2):
        A = inp.H[b].astype(np.float64) @ W1[:, :sh.d].T
        x = np.concatenate([[inp.last_tok[b]], o["tokens"][b, :-1]])
        np.testing.assert_allclose(o["u"][b], silu64(A + M[x]), rtol=0, atol=1e-12)


def test_M5_markov_brute_force_fixed_point_is_the_greedy_draft():
    """Markov head, tiny vocabulary: exactly one teacher sequence in V^(K-1) is a
    fixed point of teacher forcing, and it is the free-running greedy draft."""
    sh = small_shape(V=5, d=8, h=8, r=4, K=5)
    w = ds.make_weights(sh, (9, 50), gru_sensitive=True)
    w.W1[:, sh.d:] *= 4.0
    inp = ds.make_inputs(sh, 1, (9, 51), sigma=0.2, peak="none")
    fr = oracle.draft(w, inp.H, inp.L_base, inp.last_tok, markov=True)["tokens"][0]
    seqs = np.array(list(itertools.product(range(sh.V), repeat=sh.K - 1)), dtype=np.int32)
    teach = np.concatenate([seqs, np.zeros((len(seqs), 1), np.int32)], axis=1)
    n = len(seqs)
    out = oracle.draft(w, np.repeat(inp.H, n, 0), np.repeat(inp.L_base, n, 0), np.repeat(inp.last_tok, n),
                       teacher=teach, want_logits=False, want_state=False, threads=1, markov=True)["tokens"]
    fixed = [j for j in range(n) if np.array_equal(out[j, :sh.K - 1], seqs[j])]
    assert len(fixed) == 1
    np.testing.assert_array_equal(out[fixed[0]], fr)
    assert len({tuple(x) for x in out}) > 1
