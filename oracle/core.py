"""ctypes front end of the C oracle (domino_oracle.c).

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "domino_oracle.c")
# ORACLE_LIB names another build of the same source (the sanitizer test runs the pins
# against an -fsanitize=address,undefined build this way)
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no fast-math, no -march)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Head(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("h", ctypes.c_int32), ("r", ctypes.c_int32),
                ("V", ctypes.c_int32), ("K", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p), ("W_ih", ctypes.c_void_p),
                ("W_hh", ctypes.c_void_p), ("b_ih", ctypes.c_void_p), ("b_hh", ctypes.c_void_p),
                ("E", ctypes.c_void_p), ("markov", ctypes.c_int32)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.environ.get("ORACLE_LIB") and (not os.path.exists(_LIB) or
                                                 os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_draft_row.argtypes = [ctypes.POINTER(_Head), P, P, ctypes.c_int32, P, P, P, P, P, P, P,
                                         ctypes.c_int]
        lib.oracle_draft_row.restype = ctypes.c_int
        lib.oracle_accept_len.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P]
        lib.oracle_accept_len.restype = None
        lib.oracle_verify.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
        lib.oracle_verify.restype = None
        lib.oracle_param_count.argtypes = [ctypes.c_int64] * 4 + [ctypes.c_int32]
        lib.oracle_param_count.restype = ctypes.c_int64
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _weight_dtype(shape):
    return np.float32 if shape.wdtype == "f32" else np.uint16


def draft(weights, H, L_base, last_tok, teacher=None, S_init=None, want_logits=True, want_state=True,
          threads: Optional[int] = None, markov: bool = False):
    """Run the oracle on every row of the given arrays.

    weights: domino_synth.HeadWeights (or any object with .shape and the seven arrays)
    H [n,K,d] (weight storage dtype), L_base [n,K,V] float32, last_tok [n] int32,
    teacher [n,K] int32 or None, S_init [n,h] float32 or None.
    markov: the Markov head (every GRU step from the zero state; S_init must be None).

    Returns a dict: tokens [n,K] int32, gap [n,K] float64, flags [n] int32 and,
    when requested, L_final [n,K,V] float64, S [n,K,h] float64 (S_0..S_{K-1}),
    u [n,K,r] float64 (u_1..u_K).
    """
    lib = _load()
    sh = weights.shape
    wdt = _weight_dtype(sh)
    arrs = {}
    for name in ("W1", "W2", "W_ih", "W_hh", "b_ih", "b_hh", "E"):
        a = getattr(weights, name)
        arrs[name] = None if a is None else np.ascontiguousarray(a, dtype=wdt)
    assert not (markov and S_init is not None), "a Markov head has no initial state"
    head = _Head(sh.d, sh.h, sh.r, sh.V, sh.K, 0 if sh.wdtype == "f32" else 1,
                 *[_ptr(arrs[k]) for k in ("W1", "W2", "W_ih", "W_hh", "b_ih", "b_hh", "E")],
                 1 if markov else 0)
    H = np.ascontiguousarray(H, dtype=wdt)
    L_base = np.ascontiguousarray(L_base, dtype=np.float32)
    last_tok = np.ascontiguousarray(last_tok, dtype=np.int32)
    n = L_base.shape[0]
    K, V, h, r, d = sh.K, sh.V, sh.h, sh.r, sh.d
    assert H.shape == (n, K, d) and L_base.shape == (n, K, V) and last_tok.shape == (n,)
    if teacher is not None:
        teacher = np.ascontiguousarray(teacher, dtype=np.int32)
        assert teacher.shape == (n, K)
    if S_init is not None:
        S_init = np.ascontiguousarray(S_init, dtype=np.float32)
        assert S_init.shape == (n, h)
    nt = threads if threads is not None else max_threads()
    tokens = np.empty((n, K), np.int32)
    gap = np.empty((n, K), np.float64)
    flags = np.zeros(n, np.int32)
    Lf = np.empty((n, K, V), np.float64) if want_logits else None
    S = np.empty((n, K, h), np.float64) if want_state else None
    u = np.empty((n, K, r), np.float64) if want_state else None
    for b in range(n):
        flags[b] = lib.oracle_draft_row(
            ctypes.byref(head), _ptr(H[b]), _ptr(L_base[b]), int(last_tok[b]),
            None if teacher is None else _ptr(teacher[b]), None if S_init is None else _ptr(S_init[b]),
            _ptr(tokens[b]), None if Lf is None else _ptr(Lf[b]), _ptr(gap[b]),
            None if S is None else _ptr(S[b]), None if u is None else _ptr(u[b]), int(nt))
    out = dict(tokens=tokens, gap=gap, flags=flags)
    if want_logits:
        out["L_final"] = Lf
    if want_state:
        out["S"] = S
        out["u"] = u
    return out


def accept_len(draft_tokens, target_tokens) -> np.ndarray:
    lib = _load()
    d = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    t = np.ascontiguousarray(target_tokens, dtype=np.int32)
    assert d.shape == t.shape and d.ndim == 2
    out = np.empty(d.shape[0], np.int32)
    lib.oracle_accept_len(d.shape[0], d.shape[1], _ptr(d), _ptr(t), _ptr(out))
    return out


def verify(logits, draft_tokens) -> dict:
    """Greedy verify step: logits [B, K+1, V] float32, draft [B, K] int32.

    Returns target [B, K+1], accept [B] and next [B] (int32), see oracle_verify.
    """
    lib = _load()
    lg = np.ascontiguousarray(logits, dtype=np.float32)
    d = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    B, K = d.shape
    assert lg.ndim == 3 and lg.shape[0] == B and lg.shape[1] == K + 1
    V = lg.shape[2]
    tgt = np.empty((B, K + 1), np.int32)
    acc = np.empty(B, np.int32)
    nxt = np.empty(B, np.int32)
    lib.oracle_verify(B, K, V, _ptr(lg), _ptr(d), _ptr(tgt), _ptr(acc), _ptr(nxt))
    return dict(target=tgt, accept=acc, next=nxt)


def param_count(d: int, h: int, r: int, V: int, with_bias: bool = False) -> int:
    return int(_load().oracle_param_count(d, h, r, V, 1 if with_bias else 0))
