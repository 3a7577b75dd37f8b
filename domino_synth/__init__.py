"""Seeded synthetic inputs for the Domino head drafting loop.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no projection, no GRU, no argmax over corrected
logits), so both the fp64 oracle and the HIP path can take their inputs from
it without sharing any computation.

What the inputs stand in for.  The Domino pages (paper.oopus.info review,
section "二、核心方法与创新"; news.sig.ai article, section "Domino怎么做")
describe a parallel draft backbone that, in one forward pass, yields hidden
states H and base logits L_base for a whole 16-token block, plus a trained
Domino head (GRU causal encoder with hidden size 1024, rank-256 low-rank
correction).  No trained weights or datasets are available, so every tensor
here is a seeded draw with the shapes of the Qwen3-4B/8B-shaped heads and the
distributions stated next to each array below.

Recipe (all draws float32 from numpy's PCG64, keyed by SeedSequence):

* weights ~ N(0, 1/fan_in): fan_in = d+h for W1, r for W2, d for W_ih,
  h for W_hh and for both GRU bias vectors; the token embedding table
  E ~ N(0, 0.02^2).  Large arrays are drawn in row chunks of ``CHUNK_ROWS``,
  chunk c of array a from SeedSequence(weight_key + [a, c]), so the draw is
  the same whatever the thread count.
* per batch row b (key = row_key + [b]): H ~ N(0,1) from key+[0]; the
  L_base noise ~ N(0, sigma^2) from key+[1]; the planted peak ids from
  key+[2]; last_tok ~ U{0..V-1} from key+[3]; the temperature from key+[4].
* planted peak: for each position, L_base[v*] = max_v(noise) + peak_height,
  i.e. the planted token sits ``peak_height`` above that position's noise
  maximum.  v* is uniform (tiny head) or Zipf(s=1.1) over ranks 1..V
  (rank k -> token id k-1, ranks beyond V redrawn).
* optional per-row temperature T_b ~ U[1, 4]: the whole L_base row is
  divided by T_b after planting.
* bf16 arrays are float32 draws rounded to bfloat16 by round-to-nearest-
  even on the bit pattern and stored as ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence

import numpy as np

CHUNK_ROWS = 4096

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class HeadShape:
    """Dimensions of one Domino head.

    d: backbone hidden size (width of H and of an embedding row)
    h: GRU hidden size (the pages fix 1024 for the released heads)
    r: rank of the low-rank correction (the pages fix 256)
    V: vocabulary size
    K: block size (the pages fix 16)
    wdtype: storage type of weights, H and E ("f32" or "bf16")
    """

    d: int
    h: int
    r: int
    V: int
    K: int = 16
    wdtype: str = BF16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: HeadShape
    B: int
    weight_key: tuple
    row_key: tuple
    sigma: float = 3.0
    peak: str = "zipf"  # "zipf" | "uniform" | "none"
    peak_height: float = 6.0
    temperature: Optional[tuple] = None  # (lo, hi) or None
    gru_sensitive: bool = False


TINY = HeadShape(d=256, h=64, r=16, V=1024, K=16, wdtype=F32)
QWEN3_4B = HeadShape(d=2560, h=1024, r=256, V=151936, K=16, wdtype=BF16)
QWEN3_8B = HeadShape(d=4096, h=1024, r=256, V=151936, K=16, wdtype=BF16)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, 1, (1, 0), (1, 1), sigma=2.0, peak="uniform"),
    "qwen3_4b_b1": Workload("qwen3_4b_b1", QWEN3_4B, 1, (2, 0), (2, 1)),
    "qwen3_8b_b1": Workload("qwen3_8b_b1", QWEN3_8B, 1, (3, 0), (3, 1)),
    "qwen3_8b_b32": Workload("qwen3_8b_b32", QWEN3_8B, 32, (3, 0), (4, 1)),
    "qwen3_8b_b256": Workload("qwen3_8b_b256", QWEN3_8B, 256, (3, 0), (5, 1), temperature=(1.0, 4.0)),
}


def _rng(key: Sequence[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    NaN inputs map to a quiet NaN pattern; no draw here produces NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_rows(key, aid, rows, cols, std, wdtype):
    """rows x cols draw of N(0, std^2), chunked by CHUNK_ROWS rows."""
    nchunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    out = np.empty((rows, cols), dtype=np.float32 if wdtype == F32 else np.uint16)

    def one(c):
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        g = _rng(list(key) + [aid, c])
        buf = np.empty((r1 - r0, cols), dtype=np.float32)
        g.standard_normal(out=buf, dtype=np.float32)
        buf *= np.float32(std)
        if wdtype == F32:
            out[r0:r1] = buf
        else:
            out[r0:r1] = round_to_bf16_bits(buf)

    if nchunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


@dataclasses.dataclass
class HeadWeights:
    """Weights of one head, in storage layout (row-major, PyTorch Linear/GRUCell layout).

    W1 [r, d+h]   columns 0..d-1 multiply H_i, columns d..d+h-1 multiply S_{i-1}
    W2 [V, r]
    W_ih [3h, d]  row blocks (reset r, update z, new n)
    W_hh [3h, h]  same row blocks
    b_ih, b_hh [3h]
    E [V, d]      token embedding table
    """

    shape: HeadShape
    W1: np.ndarray
    W2: np.ndarray
    W_ih: np.ndarray
    W_hh: np.ndarray
    b_ih: np.ndarray
    b_hh: np.ndarray
    E: np.ndarray

    def arrays(self):
        return dict(W1=self.W1, W2=self.W2, W_ih=self.W_ih, W_hh=self.W_hh, b_ih=self.b_ih, b_hh=self.b_hh, E=self.E)


def make_weights(shape: HeadShape, key, gru_sensitive: bool = False) -> HeadWeights:
    d, h, r, V, wd = shape.d, shape.h, shape.r, shape.V, shape.wdtype
    W1 = _normal_rows(key, 0, r, d + h, 1.0 / np.sqrt(d + h), F32)
    if gru_sensitive:
        # stronger state columns: W1_S ~ N(0, 4/h)
        W1[:, d:] = _normal_rows(key, 10, r, h, 2.0 / np.sqrt(h), F32)
    W1 = W1 if wd == F32 else round_to_bf16_bits(W1)
    W2 = _normal_rows(key, 1, V, r, 1.0 / np.sqrt(r), wd)
    W_ih = _normal_rows(key, 2, 3 * h, d, 1.0 / np.sqrt(d), wd)
    W_hh = _normal_rows(key, 3, 3 * h, h, 1.0 / np.sqrt(h), wd)
    b_ih = _normal_rows(key, 4, 1, 3 * h, 1.0 / np.sqrt(h), wd)[0].copy()
    b_hh = _normal_rows(key, 5, 1, 3 * h, 1.0 / np.sqrt(h), wd)[0].copy()
    E = _normal_rows(key, 6, V, d, 1.0 if gru_sensitive else 0.02, wd)
    return HeadWeights(shape, W1, W2, W_ih, W_hh, b_ih, b_hh, E)


@dataclasses.dataclass
class BlockInputs:
    """Per-call inputs for B batch rows.

    H [B, K, d] (wdtype), L_base [B, K, V] float32, last_tok [B] int32,
    temperature [B] float32 (1.0 where none was applied).
    """

    H: np.ndarray
    L_base: np.ndarray
    last_tok: np.ndarray
    temperature: np.ndarray
    peak_ids: np.ndarray


def _zipf_ids(g: np.random.Generator, n: int, V: int, s: float = 1.1) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    filled = 0
    while filled < n:
        k = g.zipf(s, size=n - filled)
        k = k[k <= V]
        take = min(len(k), n - filled)
        out[filled:filled + take] = k[:take] - 1
        filled += take
    return out


def make_row(shape: HeadShape, row_key, b: int, sigma: float, peak: str, peak_height: float,
             temperature: Optional[tuple]):
    K, d, V, wd = shape.K, shape.d, shape.V, shape.wdtype
    key = list(row_key) + [b]
    gH = _rng(key + [0])
    Hf = np.empty((K, d), dtype=np.float32)
    gH.standard_normal(out=Hf, dtype=np.float32)
    H = Hf if wd == F32 else round_to_bf16_bits(Hf)
    gL = _rng(key + [1])
    L = np.empty((K, V), dtype=np.float32)
    gL.standard_normal(out=L, dtype=np.float32)
    L *= np.float32(sigma)
    gP = _rng(key + [2])
    if peak == "uniform":
        ids = gP.integers(0, V, size=K)
    elif peak == "zipf":
        ids = _zipf_ids(gP, K, V)
    else:
        ids = np.full(K, -1, dtype=np.int64)
    if peak != "none":
        top = L.max(axis=1)
        L[np.arange(K), ids] = top + np.float32(peak_height)
    last = int(_rng(key + [3]).integers(0, V))
    T = np.float32(1.0)
    if temperature is not None:
        T = np.float32(_rng(key + [4]).uniform(temperature[0], temperature[1]))
        L /= T
    return H, L, last, T, ids


def make_inputs(shape: HeadShape, rows, row_key, sigma=3.0, peak="zipf", peak_height=6.0,
                temperature=None) -> BlockInputs:
    """Inputs for the batch rows ``rows`` (an int B means rows 0..B-1).

    Each row's draw depends only on its own index, so a subset of rows of a
    large batch equals those rows of the full batch.
    """
    rows = list(range(rows)) if isinstance(rows, (int, np.integer)) else list(rows)
    n = len(rows)
    K, d, V = shape.K, shape.d, shape.V
    H = np.empty((n, K, d), dtype=np.float32 if shape.wdtype == F32 else np.uint16)
    L = np.empty((n, K, V), dtype=np.float32)
    last = np.empty(n, dtype=np.int32)
    T = np.ones(n, dtype=np.float32)
    ids = np.empty((n, K), dtype=np.int64)

    def one(j):
        H[j], L[j], last[j], T[j], ids[j] = make_row(shape, row_key, rows[j], sigma, peak, peak_height,
                                                     temperature)

    if n == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(n)))
    return BlockInputs(H, L, last, T, ids)


def make_workload(name: str, B: Optional[int] = None, rows: Optional[Sequence[int]] = None):
    """(weights, inputs) for a named workload; ``rows`` selects batch rows, ``B`` the batch size."""
    wl = WORKLOADS[name]
    w = make_weights(wl.shape, wl.weight_key, gru_sensitive=wl.gru_sensitive)
    sel = rows if rows is not None else (B if B is not None else wl.B)
    inp = make_inputs(wl.shape, sel, wl.row_key, wl.sigma, wl.peak, wl.peak_height, wl.temperature)
    return w, inp


def uniform_tokens(key, shape_, V: int) -> np.ndarray:
    return _rng(key).integers(0, V, size=shape_).astype(np.int32)


def geometric_prefix_targets(draft: np.ndarray, key, V: int, mean: float = 7.0):
    """Synthetic verifier tokens for accept-length tests.

    For row b, k_b ~ Geometric on {0,1,...} with mean ``mean`` (p = 1/(mean+1)),
    truncated to K (K when V = 1).  target[b, :k] = draft[b, :k]; if k < K, target[b, k] is a
    uniform token redrawn until it differs from draft[b, k]; positions after k
    are uniform.  Returns (target [B,K] int32, k [B] int32).
    """
    draft = np.asarray(draft, dtype=np.int32)
    B, K = draft.shape
    p = 1.0 / (mean + 1.0)
    tgt = np.empty_like(draft)
    ks = np.empty(B, dtype=np.int32)
    for b in range(B):
        g = _rng(list(key) + [b])
        k = int(g.geometric(p)) - 1  # numpy's geometric has support {1,2,...}
        k = min(k, K) if V > 1 else K  # with one token id no position can differ
        row = g.integers(0, V, size=K).astype(np.int32)
        row[:k] = draft[b, :k]
        if k < K:
            while row[k] == draft[b, k]:
                row[k] = g.integers(0, V)
        tgt[b] = row
        ks[b] = k
    return tgt, ks


@dataclasses.dataclass
class VerifyInputs:
    draft: np.ndarray    # [B, K] int32
    logits: np.ndarray   # [B, K+1, V] float32 target logits
    planted: np.ndarray  # [B, K+1] int32 token planted on top of each logits row
    k: np.ndarray        # [B] int32 planted accept length


def make_verify_inputs(B: int, K: int, V: int, key, sigma: float = 3.0, peak_height: float = 6.0,
                       mean: float = 7.0) -> VerifyInputs:
    """Inputs of the greedy verify step for B drafted blocks of K tokens.

    Row b (key + [b]): draft ~ Zipf(1.1) token ids from key+[b,0]; the target's
    tokens come from ``geometric_prefix_targets`` (key+[1]): equal to the draft
    for the first k_b positions (k_b ~ Geometric, mean ``mean``, truncated to K),
    different at position k_b, uniform afterwards, plus a uniform token for row
    K (key+[b,2]).  Each logits row is N(0, sigma^2) noise (key+[b,3]) with the
    target's token set ``peak_height`` above the row's noise maximum, the same
    planting as the base logits of the draft workloads.
    """
    draft = np.empty((B, K), np.int32)
    for b in range(B):
        draft[b] = _zipf_ids(_rng(list(key) + [b, 0]), K, V).astype(np.int32)
    tgt, ks = geometric_prefix_targets(draft, list(key) + [1], V, mean)
    planted = np.empty((B, K + 1), np.int32)
    planted[:, :K] = tgt
    logits = np.empty((B, K + 1, V), np.float32)

    def one(b):
        planted[b, K] = int(_rng(list(key) + [b, 2]).integers(0, V))
        L = logits[b]
        _rng(list(key) + [b, 3]).standard_normal(out=L, dtype=np.float32)
        L *= np.float32(sigma)
        top = L.max(axis=1)
        L[np.arange(K + 1), planted[b]] = top + np.float32(peak_height)

    if B == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(B)))
    return VerifyInputs(draft, logits, planted, ks)


def digest(*arrays) -> str:
    """Short content hash used by the determinism tests."""
    hsh = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        hsh.update(str(a.dtype).encode())
        hsh.update(str(a.shape).encode())
        hsh.update(a.tobytes())
    return hsh.hexdigest()[:16]
