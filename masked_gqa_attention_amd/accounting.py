"""Algorithmic work of one attention call, for throughput and roofline figures.

Units (the Graphcore page, "Independent attention product layouts", keeps the
valid arithmetic bounds of each product for profiling even where storage is
padded; the same rule is used here):
  * FLOPs = 4*d per visible (query row, key) pair: 2*d for the score product
    and 2*d for the probability-value product, d the logical head size.  No
    padded columns, masked pairs, skipped tiles or softmax work are counted.
  * Bytes = Q and O once each, plus every K and V row that some query row of
    the same (batch, kv head) can see, once.  Split partials, LDS traffic and
    re-reads are not counted.

Per row i (absolute key position p = i + Lkv - Lq) the visible keys form the
interval [lo, hi] with lo = max(0, p - W + 1) under a window W, hi = p under
the causal mask, or hi = min(Lkv - 1, p + W - 1) under a window without the
causal mask.
"""
from __future__ import annotations

import numpy as np


def row_intervals(Lq: int, Lkv: int, causal: bool, window: int):
    p = np.arange(Lq, dtype=np.int64) + (Lkv - Lq)
    lo = np.zeros(Lq, dtype=np.int64)
    hi = np.full(Lq, Lkv - 1, dtype=np.int64)
    if causal:
        hi = np.minimum(hi, p)
    if window > 0:
        lo = np.maximum(lo, p - window + 1)
        if not causal:
            hi = np.minimum(hi, p + window - 1)
    return lo, hi


def pairs_per_head(Lq: int, Lkv: int, causal: bool, window: int) -> int:
    lo, hi = row_intervals(Lq, Lkv, causal, window)
    return int(np.maximum(hi - lo + 1, 0).sum())


def keys_touched_per_unit(Lq: int, Lkv: int, causal: bool, window: int) -> int:
    lo, hi = row_intervals(Lq, Lkv, causal, window)
    ok = hi >= lo
    if not ok.any():
        return 0
    # Rows' intervals move monotonically with p, so their union is contiguous.
    return int(hi[ok].max() - lo[ok].min() + 1)


def work(B, Hq, Hkv, Lq, Lkv, d, causal, window, elem_bytes=2) -> dict:
    pairs = pairs_per_head(Lq, Lkv, causal, window) * B * Hq
    flops = 4 * d * pairs
    q_bytes = B * Hq * Lq * d * elem_bytes
    kv_bytes = 2 * B * Hkv * keys_touched_per_unit(Lq, Lkv, causal, window) * d * elem_bytes
    return {"pairs": pairs, "flops": flops, "bytes": 2 * q_bytes + kv_bytes,
            "q_bytes": q_bytes, "kv_bytes": kv_bytes}


def workload_work(w) -> dict:
    return work(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, w.causal, w.window)
