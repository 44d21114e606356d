"""Oracle: plain float64 CPU masked grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The product path (the
HIP library and its Python binding) never imports, calls or links it, and it
imports nothing from the product path.

What it computes (the task page "TPU v6e Masked GQA Kernel Optimization",
sections "What You Have" and "Hard Constraints"): for every batch b, query
head h and query row i,

    O[b,h,i,:] = softmax_j( mask( softcap( Q[b,h,i,:] . K[b,g,j,:] / sqrt(d) ) ) ) . V[b,g,j,:]

with g the key/value head of h under grouped-query sharing, an optional causal
mask, an optional sliding window and an optional tanh logit softcap.  The page
names the features but prints no formula, so the plainest readings are taken
(each helper says which):

* scale 1/sqrt(d) with d the logical head size;
* softcap c > 0 maps a scaled score s to c*tanh(s/c), applied before the mask;
* grouped-query sharing: G = Hq/Hkv consecutive query heads share one K/V head;
* the causal mask is aligned bottom-right: query row i sits at key position
  i + (Lkv - Lq);
* a window W > 0 keeps the W keys ending at that position (diagonal included);
  without the causal mask it keeps |pos - j| < W on both sides;
* masked keys get probability exactly 0; a row with no valid key is an error.

The method streams keys block by block with an online softmax; in exact
arithmetic that reaches the plain definition above, so the oracle is the
definition itself, materialising the full score matrix per head.
"""
from __future__ import annotations

import math

import numpy as np


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head h: consecutive groups of Hq/Hkv
    query heads share one K/V head (GQA ratios 1:1 to 16:1, task page
    "What You Have")."""
    return h // (Hq // Hkv)


def scale(d: int) -> float:
    """Score scale 1/sqrt(d), d the logical head size."""
    return 1.0 / math.sqrt(d)


def apply_softcap(s: np.ndarray, softcap: float) -> np.ndarray:
    """Tanh logit softcap c*tanh(s/c) for c > 0; identity otherwise
    (task page "What You Have": optional logit softcap)."""
    if softcap > 0:
        return softcap * np.tanh(s / softcap)
    return s


def visible(pos, j, causal: bool, window: int):
    """Elementwise visibility of key j to a query at absolute key position
    pos (arrays broadcast).  Causal: j <= pos.  Window W > 0: pos - j < W,
    and without the causal mask also j - pos < W."""
    ok = np.ones(np.broadcast(pos, j).shape, dtype=bool)
    if causal:
        ok &= j <= pos
    if window > 0:
        ok &= (pos - j) < window
        if not causal:
            ok &= (j - pos) < window
    return ok


def band(Lq: int, Lkv: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [Lq, Lkv]: True where key j is visible to query row i.
    Query row i sits at key position i + (Lkv - Lq) (bottom-right)."""
    i = np.arange(Lq)[:, None]
    j = np.arange(Lkv)[None, :]
    return visible(i + (Lkv - Lq), j, causal, window)


def band_row(i: int, Lq: int, Lkv: int, causal: bool, window: int) -> np.ndarray:
    """Row i of band(): the keys visible to query row i."""
    return visible(i + (Lkv - Lq), np.arange(Lkv), causal, window)


def softmax_masked(s: np.ndarray, ok: np.ndarray) -> np.ndarray:
    """Row softmax over the visible keys; masked keys get exactly 0.
    The row maximum is subtracted first (numerically stable form)."""
    if not ok.any(axis=-1).all():
        raise ValueError("a query row has no visible key")
    s = np.where(ok, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B,H,L,d]")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lkv, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Lq, Lkv, d


def probabilities(q, k, v, causal=False, window=0, softcap=0.0):
    """Attention probabilities P[b,h,i,j] in float64 (for invariant checks)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Hkv, Lq, Lkv, d = _check(q, k, np.asarray(v))
    ok = band(Lq, Lkv, causal, window)
    P = np.empty((B, Hq, Lq, Lkv))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            s = (q[b, h] @ k[b, g].T) * scale(d)
            s = apply_softcap(s, softcap)
            P[b, h] = softmax_masked(s, ok)
    return P


def attention(q, k, v, causal=False, window=0, softcap=0.0):
    """Full output O[B,Hq,Lq,dv] in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, Lq, Lkv, d = _check(q, k, v)
    ok = band(Lq, Lkv, causal, window)
    out = np.empty((B, Hq, Lq, v.shape[-1]))
    for b in range(B):
        for h in range(Hq):
            g = kv_head(h, Hq, Hkv)
            s = (q[b, h] @ k[b, g].T) * scale(d)
            s = apply_softcap(s, softcap)
            out[b, h] = softmax_masked(s, ok) @ v[b, g]
    return out


def attention_rows(q, k, v, rows, causal=False, window=0, softcap=0.0):
    """Output rows O[b,h,i,:] for a list of (b, h, i), one at a time, in
    float64.  Same definition as attention(); meant for sampled checks at
    sizes where the full output is too slow."""
    B, Hq, Lq, d = q.shape
    Hkv, Lkv = k.shape[1], k.shape[2]
    out = np.empty((len(rows), v.shape[-1]))
    for n, (b, h, i) in enumerate(rows):
        g = kv_head(h, Hq, Hkv)
        qi = np.asarray(q[b, h, i], dtype=np.float64)
        kk = np.asarray(k[b, g], dtype=np.float64)
        vv = np.asarray(v[b, g], dtype=np.float64)
        ok = band_row(i, Lq, Lkv, causal, window)
        s = (kk @ qi) * scale(d)
        s = apply_softcap(s, softcap)
        out[n] = softmax_masked(s[None, :], ok[None, :])[0] @ vv
    return out


def visible_pairs(Lq: int, Lkv: int, causal: bool, window: int) -> int:
    """Number of (query row, key) pairs inside the band for one head,
    counted from the mask itself."""
    return int(band(Lq, Lkv, causal, window).sum())
