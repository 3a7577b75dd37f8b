"""ctypes binding of libdomino_head.so.

Argument marshalling only: every step of the draft runs in the HIP library.
PyTorch supplies device memory (tensors) and the current HIP stream.  If the
library has not been built, loading fails with an error instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# DOMINO_LIB names another build of the same sources (the host-sanitizer test uses it)
LIB_PATH = os.environ.get("DOMINO_LIB") or os.path.join(HERE, "libdomino_head.so")

DOMINO_F32 = 0
DOMINO_BF16 = 1
EXEC_AUTO = 0
EXEC_PERSISTENT = 1
EXEC_STEPWISE = 2
FOLD_EMBED = 4
EXEC_STREAM_W2 = 8
EXEC_PLAIN_LAUNCH = 16
EXEC_POSITION_BATCHED = 32
LBASE_BF16 = 64
MARKOV = 128
FLAG_BAD_TOKEN = 1
FLAG_SYNC_TIMEOUT = 2

ERRORS = {-1: "EINVAL", -2: "EUNSUPPORTED", -3: "EWORKSPACE", -4: "EHIP", -5: "EDEVICE"}

SYMBOLS = ("domino_head_workspace_size", "domino_head_create", "domino_head_draft", "domino_accept_len",
           "domino_verify_workspace_size", "domino_verify", "domino_verify_noalloc", "domino_head_check_error", "domino_head_exec_info",
           "domino_head_set_spin_limit", "domino_head_param_count", "domino_head_destroy", "domino_last_error")


class DominoError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("h", ctypes.c_int32), ("r", ctypes.c_int32), ("V", ctypes.c_int32),
                ("K", ctypes.c_int32), ("max_batch", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("W1", ctypes.c_void_p), ("W2", ctypes.c_void_p),
                ("W_ih", ctypes.c_void_p), ("W_hh", ctypes.c_void_p), ("b_ih", ctypes.c_void_p),
                ("b_hh", ctypes.c_void_p), ("E", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libdomino_head.so is not built (%s); build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`" % path)
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.domino_head_workspace_size.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_size_t)]
    lib.domino_head_create.argtypes = [ctypes.POINTER(Config), P, ctypes.c_size_t, ctypes.POINTER(P)]
    lib.domino_head_draft.argtypes = [P, I32, P, P, P, P, P, P, P, P, P, P]
    lib.domino_accept_len.argtypes = [I32, I32, P, P, P, P]
    lib.domino_verify_workspace_size.argtypes = [I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)]
    lib.domino_verify.argtypes = [I32, I32, I32, P, P, P, ctypes.c_size_t, P, P, P, P]
    lib.domino_verify_noalloc.argtypes = [I32, I32, I32, P, P, P, P, P, P]
    lib.domino_head_check_error.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    PI = ctypes.POINTER(ctypes.c_int32)
    lib.domino_head_exec_info.argtypes = [P, I32, PI, PI, PI]
    lib.domino_head_set_spin_limit.argtypes = [P, ctypes.c_uint32]
    lib.domino_head_param_count.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_int64)]
    lib.domino_head_destroy.argtypes = [P]
    lib.domino_head_destroy.restype = None
    lib.domino_last_error.argtypes = []
    lib.domino_last_error.restype = ctypes.c_char_p
    for name in SYMBOLS[:-2]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise DominoError(rc, load_library().domino_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _weight_dtype(wdtype: int):
    return torch.float32 if wdtype == DOMINO_F32 else torch.bfloat16


class DominoHead:
    """A Domino head bound to borrowed device weights.

    fold_embedding: precompute the folded input-gate table P = E W_ih^T + b_ih ([V, 3h] float32 in the
    workspace) once, so each GRU step gathers a row of P instead of a W_ih matrix-vector product.

    markov: the Markov head (DOMINO_MARKOV): each position's state is the GRU step on the preceding
    token from the zero state, S_p = GRU(E[x_p], 0), gathered from a per-token table filled at create.
    Such a head takes no S_init and returns no S (``want_state`` then gives u only).

    weights: dict with W1 [r,d+h], W2 [V,r], W_ih [3h,d], W_hh [3h,h], b_ih/b_hh [3h] (or None) and
    E [V,d], all contiguous CUDA tensors of one dtype (float32 or bfloat16).  The tensors must stay
    alive and unmodified while the head exists (the object keeps references).
    """

    def __init__(self, weights: dict, K: int = 16, max_batch: int = 1, exec_mode: int = EXEC_AUTO,
                 fold_embedding: bool = False, lbase_bf16: bool = False, markov: bool = False):
        lib = load_library()
        W1 = weights["W1"]
        wdtype = DOMINO_F32 if W1.dtype == torch.float32 else DOMINO_BF16
        want = _weight_dtype(wdtype)
        for k in ("W1", "W2", "W_ih", "W_hh", "b_ih", "b_hh", "E"):
            t = weights.get(k)
            if t is None and k in ("b_ih", "b_hh"):
                continue
            if t is None or not t.is_cuda or t.dtype != want or not t.is_contiguous():
                raise ValueError("%s must be a contiguous CUDA tensor of dtype %s" % (k, want))
        r, dh = W1.shape
        V = weights["W2"].shape[0]
        h = weights["W_hh"].shape[1]
        d = weights["E"].shape[1]
        if dh != d + h:
            raise ValueError("W1 has %d columns, expected d+h = %d" % (dh, d + h))
        self.d, self.h, self.r, self.V, self.K = d, h, r, V, K
        self.max_batch = max_batch
        self.wdtype = wdtype
        self._weights = dict(weights)
        self.lbase_dtype = torch.bfloat16 if lbase_bf16 else torch.float32
        self.markov = markov
        flags = (exec_mode | (FOLD_EMBED if fold_embedding else 0) | (LBASE_BF16 if lbase_bf16 else 0) |
                 (MARKOV if markov else 0))
        self.cfg = Config(d, h, r, V, K, max_batch, wdtype, flags, _ptr(W1), _ptr(weights["W2"]),
                          _ptr(weights["W_ih"]), _ptr(weights["W_hh"]), _ptr(weights.get("b_ih")),
                          _ptr(weights.get("b_hh")), _ptr(weights["E"]))
        nbytes = ctypes.c_size_t()
        _check(lib.domino_head_workspace_size(ctypes.byref(self.cfg), ctypes.byref(nbytes)))
        self.workspace_bytes = int(nbytes.value)
        raw = torch.empty(self.workspace_bytes + 256, dtype=torch.uint8, device=W1.device)
        off = (-raw.data_ptr()) % 256
        self._ws_raw = raw
        self.workspace = raw[off:off + self.workspace_bytes]
        handle = ctypes.c_void_p()
        _check(lib.domino_head_create(ctypes.byref(self.cfg), _ptr(self.workspace), self.workspace_bytes,
                                      ctypes.byref(handle)))
        self._h = handle
        self.device = W1.device

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.domino_head_destroy(h)
            self._h = None

    def param_count(self) -> int:
        n = ctypes.c_int64()
        _check(load_library().domino_head_param_count(ctypes.byref(self.cfg), ctypes.byref(n)))
        return int(n.value)

    def draft(self, H: torch.Tensor, L_base: torch.Tensor, last_tok: torch.Tensor, teacher=None, S_init=None,
              want_logits: bool = False, want_state: bool = False, out: Optional[dict] = None) -> dict:
        """Greedy draft of one block for B rows, asynchronous on the current stream.

        Returns a dict with tokens [B,K] int32 and, when requested, L_final [B,K,V], S [B,K,h],
        u [B,K,r] (float32).  ``out`` may supply preallocated output tensors under the same keys.
        """
        B = int(L_base.shape[0])
        dev = self.device
        out = {} if out is None else dict(out)
        if "tokens" not in out:
            out["tokens"] = torch.empty((B, self.K), dtype=torch.int32, device=dev)
        if want_logits and "L_final" not in out:
            out["L_final"] = torch.empty((B, self.K, self.V), dtype=torch.float32, device=dev)
        if want_state:
            if "S" not in out and not self.markov:
                out["S"] = torch.empty((B, self.K, self.h), dtype=torch.float32, device=dev)
            if "u" not in out:
                out["u"] = torch.empty((B, self.K, self.r), dtype=torch.float32, device=dev)
        self._check_tensor("H", H, (B, self.K, self.d), _weight_dtype(self.wdtype))
        self._check_tensor("L_base", L_base, (B, self.K, self.V), self.lbase_dtype)
        self._check_tensor("last_tok", last_tok, (B,), torch.int32)
        if teacher is not None:
            self._check_tensor("teacher", teacher, (B, self.K), torch.int32)
        if S_init is not None:
            self._check_tensor("S_init", S_init, (B, self.h), torch.float32)
        # the kernels write these through raw pointers: a short or mistyped buffer would be overrun
        shapes = {"tokens": ((B, self.K), torch.int32), "L_final": ((B, self.K, self.V), torch.float32),
                  "S": ((B, self.K, self.h), torch.float32), "u": ((B, self.K, self.r), torch.float32)}
        for k, t in out.items():
            if k not in shapes:
                raise ValueError("out: unknown entry %r (expected tokens, L_final, S, u)" % k)
            if k == "S" and self.markov:
                raise ValueError("out: a Markov head returns no S")
            self._check_tensor("out[%r]" % k, t, *shapes[k])
        _check(load_library().domino_head_draft(
            self._h, B, _ptr(H), _ptr(L_base), _ptr(last_tok), _ptr(teacher), _ptr(S_init), _ptr(out["tokens"]),
            _ptr(out.get("L_final")), _ptr(out.get("S")), _ptr(out.get("u")), _stream_handle()))
        return out

    def exec_info(self, B: int = None) -> dict:
        """Launch a draft of B rows takes: {"persistent", "w2_resident", "grid"} (host only)."""
        B = self.max_batch if B is None else B
        v = [ctypes.c_int32() for _ in range(3)]
        _check(load_library().domino_head_exec_info(self._h, B, *[ctypes.byref(x) for x in v]))
        return {"persistent": bool(v[0].value), "w2_resident": bool(v[1].value), "grid": int(v[2].value)}

    def set_spin_limit(self, limit: int):
        """Bound on the device-side waits of later drafts (0 forces the timeout path)."""
        _check(load_library().domino_head_set_spin_limit(self._h, int(limit)))

    def check_error(self) -> int:
        """Synchronize, return and clear the device flags (raises DominoError if any is set)."""
        f = ctypes.c_uint32()
        rc = load_library().domino_head_check_error(self._h, ctypes.byref(f))
        if rc != 0 and rc != -5:
            _check(rc)
        return int(f.value)

    def _check_tensor(self, name, t, shape, dtype):
        if (not isinstance(t, torch.Tensor) or t.dtype != dtype or tuple(t.shape) != tuple(shape) or
                t.device != self.device or not t.is_contiguous()):
            raise ValueError("%s: expected a contiguous %s tensor on %s of shape %s, got %s" %
                             (name, dtype, self.device, shape,
                              "%s %s on %s" % (t.dtype, tuple(t.shape), t.device) if isinstance(t, torch.Tensor)
                              else type(t).__name__))


def accept_len(draft: torch.Tensor, target: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-row accepted prefix length of `draft` against `target` ([B,K] int32 CUDA tensors)."""
    if draft.shape != target.shape or draft.dim() != 2:
        raise ValueError("draft and target must both be [B,K]")
    B, K = draft.shape
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=draft.device)
    for t in (draft, target, out):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("accept_len takes contiguous CUDA int32 tensors")
    _check(load_library().domino_accept_len(B, K, _ptr(draft), _ptr(target), _ptr(out), _stream_handle()))
    return out


def verify_workspace_size(B: int, K: int, V: int) -> int:
    """Bytes of device workspace `verify` needs for B blocks of K tokens over V (host only)."""
    n = ctypes.c_size_t()
    _check(load_library().domino_verify_workspace_size(B, K, V, ctypes.byref(n)))
    return int(n.value)


def verify(logits: torch.Tensor, draft: torch.Tensor, workspace: Optional[torch.Tensor] = None,
           want_target: bool = True, out: Optional[dict] = None) -> dict:
    """Greedy verify step, asynchronous on the current stream.

    logits [B, K+1, V] float32 and draft [B, K] int32 (contiguous CUDA tensors).  Returns
    {"accept": [B], "next": [B]} (int32) and, with want_target, {"target": [B, K+1]}.
    ``workspace`` (uint8, at least verify_workspace_size bytes) and ``out`` may be preallocated.
    """
    if logits.dim() != 3 or draft.dim() != 2 or logits.shape[0] != draft.shape[0] or \
            logits.shape[1] != draft.shape[1] + 1:
        raise ValueError("logits must be [B, K+1, V] and draft [B, K]")
    B, K = draft.shape
    V = logits.shape[2]
    for name, t, dt in (("logits", logits, torch.float32), ("draft", draft, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: expected a contiguous CUDA %s tensor" % (name, dt))
    dev = logits.device
    need = verify_workspace_size(B, K, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    out = {} if out is None else dict(out)
    out.setdefault("accept", torch.empty(B, dtype=torch.int32, device=dev))
    out.setdefault("next", torch.empty(B, dtype=torch.int32, device=dev))
    if want_target:
        out.setdefault("target", torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    _check(load_library().domino_verify(B, K, V, _ptr(logits), _ptr(draft), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(out.get("target")),
                                        _ptr(out["accept"]), _ptr(out["next"]), _stream_handle()))
    return out


def verify_noalloc(logits: torch.Tensor, draft: torch.Tensor, want_target: bool = True,
                   out: Optional[dict] = None) -> dict:
    """verify() through the entry point that allocates nothing: the library's static
    scratch stands in for the workspace (at most 1 MiB of it; calls that overlap on
    one device race).  Output tensors are allocated here unless ``out`` gives them."""
    if logits.dim() != 3 or draft.dim() != 2 or logits.shape[0] != draft.shape[0] or \
            logits.shape[1] != draft.shape[1] + 1:
        raise ValueError("logits must be [B, K+1, V] and draft [B, K]")
    B, K = draft.shape
    for name, t, dt in (("logits", logits, torch.float32), ("draft", draft, torch.int32)):
        if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s: expected a contiguous CUDA %s tensor" % (name, dt))
    dev = logits.device
    out = {} if out is None else dict(out)
    out.setdefault("accept", torch.empty(B, dtype=torch.int32, device=dev))
    out.setdefault("next", torch.empty(B, dtype=torch.int32, device=dev))
    if want_target:
        out.setdefault("target", torch.empty((B, K + 1), dtype=torch.int32, device=dev))
    _check(load_library().domino_verify_noalloc(B, K, logits.shape[2], _ptr(logits), _ptr(draft),
                                                _ptr(out.get("target")), _ptr(out["accept"]), _ptr(out["next"]),
                                                _stream_handle()))
    return out
