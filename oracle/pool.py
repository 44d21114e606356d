"""Process-pool driver of the float64 oracle (TEST INFRASTRUCTURE ONLY).

Runs oracle.attention on slices of (batch row, group of query heads sharing
one K/V head) in worker processes and assembles the full output.  The
definition is per (b, h) already (the task page "TPU v6e Masked GQA Kernel
Optimization", "What You Have": every query head attends over its group's
key/value head), so each worker computes
exactly what attention() computes for those heads: the same score matrices,
the same mask, the same softmax, in the same float64 operations.  Nothing is
blocked, fused or reordered; only the loop over (b, h) is spread over
processes.

Workers are started with the "spawn" method (fresh interpreters that import
numpy and this package only), so a caller that has initialised a GPU is
never forked.  Each worker uses one BLAS thread.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time

import numpy as np

from .attention_fp64 import attention


def host_cores() -> int:
    """CPU cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _init_worker():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _heads(args):
    qh, kg, vg, causal, window, softcap = args
    return attention(qh, kg, vg, causal, window, softcap)


def _tasks(q, k, v, causal, window, softcap, workers):
    """(query heads h0..h1 of one batch row, their K/V head) slices: a unit's
    K/V travel to a worker once per task, and a unit's heads are split only as
    far as needed to give every worker a task."""
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    per_unit = min(G, max(1, -(-workers // (B * Hkv))))
    step = -(-G // per_unit)
    for b in range(B):
        for g in range(Hkv):
            for h0 in range(g * G, (g + 1) * G, step):
                h1 = min(h0 + step, (g + 1) * G)
                yield (h0, h1), (q[b:b + 1, h0:h1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                 causal, window, softcap)


class OraclePool:
    """A pool of `workers` oracle processes (default: every host core)."""

    def __init__(self, workers: int | None = None):
        self.workers = workers or host_cores()
        ctx = mp.get_context("spawn")
        env_threads = os.environ.get("OMP_NUM_THREADS")
        os.environ["OMP_NUM_THREADS"] = "1"  # inherited by the spawned workers
        try:
            self._pool = ctx.Pool(self.workers, initializer=_init_worker)
        finally:
            if env_threads is None:
                os.environ.pop("OMP_NUM_THREADS", None)
            else:
                os.environ["OMP_NUM_THREADS"] = env_threads

    def attention(self, q, k, v, causal=False, window=0, softcap=0.0) -> np.ndarray:
        """oracle.attention(q, k, v, ...) computed head by head in the pool."""
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        B, Hq, Lq = q.shape[:3]
        tasks = list(_tasks(q, k, v, causal, window, softcap, self.workers))
        parts = self._pool.map(_heads, [t for _, t in tasks], chunksize=1)
        out = np.empty((B, Hq, Lq, v.shape[-1]))
        per_batch = len(tasks) // B
        for n, ((h0, h1), o) in enumerate(zip((hs for hs, _ in tasks), parts)):
            out[n // per_batch, h0:h1] = o[0]
        return out

    def timed_attention(self, q, k, v, causal=False, window=0, softcap=0.0):
        """(output, wall seconds) of one pooled oracle run."""
        t0 = time.perf_counter()
        out = self.attention(q, k, v, causal, window, softcap)
        return out, time.perf_counter() - t0

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
