"""Seeded synthetic inputs and the named workloads.

This module is shared by the tests, the benchmark and the oracle's callers.
It holds no attention arithmetic: only random draws, the bf16/fp16 storage
formats and the workload table.  The workloads stand in for the visible and
held-out "strata" of the TPU v6e task page ("What You Have": decode, prefill
and encoder shapes, GQA 1:1 to 16:1, optional causal mask, sliding window and
logit softcap, bf16 inputs) and for the SigLIP shape of the Graphcore page
("SigLIP batch-1 hardware results": 16 heads, 729 tokens, 72 per head).

Recipe: numpy PCG64 generator seeded with the workload seed; Q, then K, then V
drawn as float32 standard normals times sigma, then rounded to the storage
type (bf16 by round-to-nearest-even on the float32 bits, fp16 by numpy's cast).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  NaN stays NaN (quiet bit set).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    bits = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        bits[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return bits


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def storage_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a storage array ("bf16" bits or "fp16")."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    if dtype == "fp16":
        return np.asarray(arr, dtype=np.float16).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def f32_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lkv: int
    d: int
    causal: bool = False
    window: int = 0          # 0: no window
    softcap: float = 0.0     # 0: no softcap
    sigma: float = 1.0
    seed: int = 0
    dtype: str = "bf16"

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def describe(self) -> dict:
        return {
            "workload": self.name, "B": self.B, "Hq": self.Hq, "Hkv": self.Hkv,
            "Lq": self.Lq, "Lkv": self.Lkv, "d": self.d, "causal": self.causal,
            "window": self.window, "softcap": self.softcap, "sigma": self.sigma,
            "seed": self.seed, "dtype": self.dtype,
        }


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_causal_gqa4_L64", B=1, Hq=4, Hkv=1, Lq=64, Lkv=64, d=128,
                 causal=True, seed=0),
        Workload("decode_gqa4_kv8192", B=8, Hq=32, Hkv=8, Lq=1, Lkv=8192, d=128,
                 causal=True, seed=1),
        Workload("prefill_gqa8_L4096_w1024_cap50", B=2, Hq=32, Hkv=4, Lq=4096,
                 Lkv=4096, d=128, causal=True, window=1024, softcap=50.0, seed=2),
        Workload("encoder_siglip_L729_d72", B=1, Hq=16, Hkv=16, Lq=729, Lkv=729,
                 d=72, causal=False, seed=3, dtype="fp16"),
        Workload("decode_gqa16_kv32768_w4096_cap30", B=4, Hq=64, Hkv=4, Lq=1,
                 Lkv=32768, d=128, causal=True, window=4096, softcap=30.0,
                 sigma=0.5, seed=4),
    ]
}

# Order in which the workloads are listed everywhere (reports, tests).
WORKLOAD_ORDER = list(WORKLOADS)

# Shapes for the extensions beyond the five workloads: a multi-token decode
# (4 new query positions per sequence, bottom-right causal), encoders with few
# heads -- at 729 tokens (the short-band kernel: each workgroup's eight waves
# split the key band among themselves) and at 1000 tokens (a band too long for
# it: the key axis split across workgroups) -- and the long windowed decode
# over a ring buffer of exactly the window's 4096 slots (ring start 1234; the
# ring's Lkv is its slot count).
NEXT_WORKLOADS = {
    w.name: w
    for w in [
        Workload("multitoken_decode_gqa4_Lq4_kv8192", B=8, Hq=32, Hkv=8, Lq=4, Lkv=8192, d=128,
                 causal=True, seed=5),
        Workload("encoder_fewheads_h4_L729_d72", B=1, Hq=4, Hkv=4, Lq=729, Lkv=729, d=72,
                 causal=False, seed=6, dtype="fp16"),
        Workload("encoder_splitk_h4_L1000_d72", B=1, Hq=4, Hkv=4, Lq=1000, Lkv=1000, d=72,
                 causal=False, seed=8, dtype="fp16"),
        Workload("ring_decode_gqa16_S4096_w4096_cap30", B=4, Hq=64, Hkv=4, Lq=1, Lkv=4096, d=128,
                 causal=True, window=4096, softcap=30.0, sigma=0.5, seed=7),
    ]
}
RING_START = 1234


def draw_qkv(w: Workload):
    """Draw Q, K, V for a workload.  Returns storage arrays (uint16 bf16 bits
    or float16), shaped [B,Hq,Lq,d], [B,Hkv,Lkv,d], [B,Hkv,Lkv,d]."""
    rng = np.random.default_rng(w.seed)
    shapes = [(w.B, w.Hq, w.Lq, w.d), (w.B, w.Hkv, w.Lkv, w.d), (w.B, w.Hkv, w.Lkv, w.d)]
    out = []
    for shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32)
        if w.sigma != 1.0:
            x *= np.float32(w.sigma)
        out.append(f32_to_storage(x, w.dtype))
    return tuple(out)


def draw_array(seed: int, shape, dtype: str = "bf16", sigma: float = 1.0) -> np.ndarray:
    """One seeded array in a storage type (for structured test inputs)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_storage(x, dtype)
