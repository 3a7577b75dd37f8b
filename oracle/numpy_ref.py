"""Vectorised NumPy float64 rewrite of the Domino head drafting loop.

TEST INFRASTRUCTURE ONLY.  Written independently of domino_oracle.c and used
solely to cross-check it on small shapes; it is not a pin of the method (the
pins are closed forms, library routines and brute force in the tests).

Same readings as the C oracle (PyTorch GRUCell gate order r, z, n; SiLU;
anchor step on last_tok; lowest-index argmax on float32-rounded logits).
Unlike the C oracle it evaluates W1 [H_i; S] as W1[:, :d] H_i + W1[:, d:] S
with matrix products, so agreement also checks that split.
"""
from __future__ import annotations

import numpy as np


def _f64(a, wdtype):
    a = np.asarray(a)
    if wdtype == "f32":
        return a.astype(np.float64)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _gru(x, s, W_ih, W_hh, b_ih, b_hh, h):
    g = W_ih @ x + b_ih
    q = W_hh @ s + b_hh
    r = 1.0 / (1.0 + np.exp(-(g[:h] + q[:h])))
    z = 1.0 / (1.0 + np.exp(-(g[h:2 * h] + q[h:2 * h])))
    n = np.tanh(g[2 * h:] + r * q[2 * h:])
    return (1.0 - z) * n + z * s


def _argmax_f32(row64):
    f = row64.astype(np.float32)
    nan = np.isnan(f)
    if nan.any():
        return int(np.flatnonzero(nan)[0])
    return int(np.argmax(f))  # first maximum


def draft(weights, H, L_base, last_tok, teacher=None, S_init=None):
    sh = weights.shape
    wd = sh.wdtype
    d, h, V, K = sh.d, sh.h, sh.V, sh.K
    W1 = _f64(weights.W1, wd)
    W2 = _f64(weights.W2, wd)
    W_ih = _f64(weights.W_ih, wd)
    W_hh = _f64(weights.W_hh, wd)
    b_ih = np.zeros(3 * h) if weights.b_ih is None else _f64(weights.b_ih, wd)
    b_hh = np.zeros(3 * h) if weights.b_hh is None else _f64(weights.b_hh, wd)
    E = weights.E
    n = len(last_tok)
    tokens = np.empty((n, K), np.int32)
    Lf = np.empty((n, K, V))
    S_all = np.empty((n, K, h))
    for b in range(n):
        Hb = _f64(H[b], wd)                      # [K, d]
        A = Hb @ W1[:, :d].T                     # [K, r]
        s = np.zeros(h) if S_init is None else np.asarray(S_init[b], np.float64)
        s = _gru(_f64(E[last_tok[b]], wd), s, W_ih, W_hh, b_ih, b_hh, h)
        for i in range(K):
            S_all[b, i] = s
            a = A[i] + W1[:, d:] @ s
            u = a / (1.0 + np.exp(-a))
            lf = L_base[b, i].astype(np.float64) + W2 @ u
            Lf[b, i] = lf
            t = _argmax_f32(lf)
            tokens[b, i] = t
            if i + 1 < K:
                x_tok = t if teacher is None else int(teacher[b, i])
                s = _gru(_f64(E[x_tok], wd), s, W_ih, W_hh, b_ih, b_hh, h)
    return dict(tokens=tokens, L_final=Lf, S=S_all)
