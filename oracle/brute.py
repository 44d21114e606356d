"""Brute-force scalar attention in pure Python, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (same rule as the float64 oracle): it exists to pin
the oracle.  It is written independently of oracle/attention_fp64.py: explicit
loops, math.exp / math.tanh, the visibility test spelled out per pair, and
no numpy arithmetic, so a slip in the vectorised oracle (an index, a sign, a
transposed operand) shows up as a disagreement.

Definition followed: the task page "TPU v6e Masked GQA Kernel Optimization"
("What You Have" lists decode/prefill/encoder shapes, GQA ratios, optional
causal mask, sliding window and logit softcap); readings as stated in the
oracle's header (bottom-right causal, window of W keys including the
diagonal, softcap c*tanh(s/c) before the mask, 1/sqrt(d) scale).
"""
from __future__ import annotations

import math


def _visible(i, j, Lq, Lkv, causal, window):
    pos = Lkv - Lq + i          # absolute key position of query row i
    if causal and j > pos:
        return False
    if window > 0:
        dist = pos - j
        if causal:
            if dist >= window:
                return False
        elif abs(dist) >= window:
            return False
    return True


def attention_brute(q, k, v, causal=False, window=0, softcap=0.0):
    """q: nested lists [B][Hq][Lq][d]; k, v: [B][Hkv][Lkv][d].
    Returns nested lists [B][Hq][Lq][dv] of Python floats."""
    B = len(q)
    Hq = len(q[0])
    Lq = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k[0])
    Lkv = len(k[0][0])
    dv = len(v[0][0][0])
    group = Hq // Hkv
    out = []
    for b in range(B):
        ob = []
        for h in range(Hq):
            g = h // group
            oh = []
            for i in range(Lq):
                scores = []
                for j in range(Lkv):
                    if not _visible(i, j, Lq, Lkv, causal, window):
                        continue
                    dot = 0.0
                    for t in range(d):
                        dot += float(q[b][h][i][t]) * float(k[b][g][j][t])
                    s = dot / math.sqrt(d)
                    if softcap > 0:
                        s = softcap * math.tanh(s / softcap)
                    scores.append((j, s))
                if not scores:
                    raise ValueError("empty row")
                top = max(s for _, s in scores)
                weights = [(j, math.exp(s - top)) for j, s in scores]
                total = math.fsum(w for _, w in weights)
                row = []
                for t in range(dv):
                    row.append(math.fsum(w * float(v[b][g][j][t]) for j, w in weights) / total)
                oh.append(row)
            ob.append(oh)
        out.append(ob)
    return out
