"""Parity cases shared by the GPU parity tests and the CPU control that feeds
planted oracle mutants through the same comparator.

Each case is a seeded synthetic problem (synth.draw_array) plus an optional
structure applied to the drawn inputs: scaled ("hot") queries that make the
softcap matter, zero queries with one-hot values that read the mask out, and
constant values.  Sizes are small enough for the float64 oracle to finish in
seconds yet span several key tiles and a ragged tail.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from masked_gqa_attention_amd import synth

RTOL = 2e-2   # tolerance stated on the task page ("Hard Constraints")
ATOL = 2e-2


@dataclass(frozen=True)
class Case:
    name: str
    B: int
    Hq: int
    Hkv: int
    Lq: int
    Lkv: int
    d: int
    causal: bool = False
    window: int = 0
    softcap: float = 0.0
    dtype: str = "bf16"
    kind: str = "normal"   # normal | hot | onehot | const
    seed: int = 100
    qscale: float = 1.0


def make_inputs(c: Case):
    """Storage arrays (bf16 bits or fp16) for q, k, v."""
    q = synth.draw_array(c.seed, (c.B, c.Hq, c.Lq, c.d), c.dtype)
    k = synth.draw_array(c.seed + 1, (c.B, c.Hkv, c.Lkv, c.d), c.dtype)
    v = synth.draw_array(c.seed + 2, (c.B, c.Hkv, c.Lkv, c.d), c.dtype)
    if c.kind == "hot":
        qf = synth.storage_to_f64(q, c.dtype) * c.qscale
        q = synth.f32_to_storage(qf.astype(np.float32), c.dtype)
    elif c.kind == "onehot":
        assert c.Lkv <= c.d
        q = synth.f32_to_storage(np.zeros((c.B, c.Hq, c.Lq, c.d), np.float32), c.dtype)
        eye = np.zeros((c.B, c.Hkv, c.Lkv, c.d), np.float32)
        for j in range(c.Lkv):
            eye[:, :, j, j] = 1.0
        v = synth.f32_to_storage(eye, c.dtype)
    elif c.kind == "const":
        v = synth.f32_to_storage(np.full((c.B, c.Hkv, c.Lkv, c.d), 0.8125, np.float32), c.dtype)
    return q, k, v


def as_f64(c: Case, arrs):
    return tuple(synth.storage_to_f64(a, c.dtype) for a in arrs)


def compare(got: np.ndarray, ref: np.ndarray, rtol=RTOL, atol=ATOL):
    """Elementwise |got-ref| <= atol + rtol*|ref| on every element, no NaN/inf.
    Returns (ok, stats)."""
    finite = bool(np.isfinite(got).all())
    err = np.abs(got - ref)
    ok = finite and bool((err <= atol + rtol * np.abs(ref)).all())
    rms_ref = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    stats = {
        "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float((err / np.maximum(np.abs(ref), 1e-6)).max()) if err.size else 0.0,
        "nrmse": float(np.sqrt(np.mean(err ** 2)) / rms_ref) if err.size else 0.0,
        "finite": finite,
    }
    return ok, stats


CASES = [
    # prefill / encoder path, ragged tails, every GQA ratio class
    Case("prefill_causal_g4_L200", 1, 8, 2, 200, 200, 128, causal=True, seed=10),
    Case("prefill_causal_g8_bottomright", 2, 16, 2, 100, 333, 128, causal=True, seed=11),
    Case("prefill_window_cap_g8", 1, 16, 2, 300, 300, 128, causal=True, window=70, softcap=20.0, seed=12),
    Case("prefill_noncausal_g1_d72", 1, 3, 3, 150, 150, 72, seed=13),
    Case("prefill_noncausal_window_g2", 1, 4, 2, 190, 190, 64, window=33, seed=14),
    Case("prefill_g3_d96", 1, 6, 2, 77, 130, 96, causal=True, seed=15),
    Case("prefill_g16_d64", 1, 32, 2, 40, 70, 64, causal=True, window=17, seed=16),
    Case("prefill_fp16_d72", 1, 4, 4, 129, 129, 72, dtype="fp16", seed=17),
    Case("prefill_noncausal_longq", 1, 2, 1, 150, 90, 128, seed=18),
    Case("prefill_d8", 1, 2, 1, 70, 70, 8, causal=True, seed=19),
    Case("prefill_d32_g2", 1, 4, 2, 65, 65, 32, causal=True, window=9, seed=20),
    Case("prefill_window1", 1, 2, 1, 100, 100, 128, causal=True, window=1, seed=21),
    # decode path (G*Lq <= 16), splits, multi-token rows
    Case("decode_g4_kv3000", 2, 8, 2, 1, 3000, 128, causal=True, seed=30),
    Case("decode_g16_window_cap", 1, 32, 2, 1, 2500, 128, causal=True, window=700, softcap=30.0, seed=31),
    Case("decode_g1_noncausal_d72", 2, 2, 2, 1, 1000, 72, seed=32),
    Case("decode_multitoken_g4_lq3", 1, 8, 2, 3, 1500, 128, causal=True, window=300, seed=33),
    Case("decode_multitoken_g2_lq8", 1, 4, 2, 8, 600, 64, causal=True, seed=34),
    Case("decode_short_kv", 1, 16, 1, 1, 37, 128, causal=True, seed=35),
    Case("decode_fp16", 1, 8, 1, 1, 900, 128, causal=True, dtype="fp16", seed=36),
    Case("decode_window_edge", 1, 4, 1, 1, 1030, 128, causal=True, window=129, seed=37),
    # structured inputs
    Case("hot_softcap_prefill", 1, 8, 2, 130, 130, 128, causal=True, softcap=50.0, kind="hot", qscale=8.0, seed=40),
    Case("hot_softcap_decode", 1, 16, 1, 1, 800, 128, causal=True, softcap=30.0, kind="hot", qscale=8.0, seed=41),
    Case("hot_noscale_prefill", 1, 4, 1, 100, 100, 128, causal=True, kind="hot", qscale=20.0, seed=42),
    Case("onehot_causal_window", 1, 4, 2, 100, 120, 128, causal=True, window=7, kind="onehot", seed=43),
    Case("onehot_noncausal_window", 1, 2, 1, 64, 64, 64, window=5, kind="onehot", seed=44),
    Case("onehot_decode_window", 1, 8, 1, 1, 128, 128, causal=True, window=50, kind="onehot", seed=45),
    Case("const_v_prefill", 1, 8, 2, 90, 90, 72, causal=True, window=20, softcap=5.0, kind="const", seed=46),
    Case("const_v_decode", 1, 4, 1, 2, 700, 128, causal=True, kind="const", seed=47),
    # split-KV kernel with several 16-row blocks per workgroup (position blocks
    # of 16*nqb/G positions), with and without key splits across workgroups
    Case("split_nqb4_d64_g2", 2, 16, 8, 512, 600, 64, causal=True, seed=50),
    Case("split_nqb3_d72_fp16", 1, 18, 18, 700, 700, 72, dtype="fp16", seed=51),
    Case("split_nqb2_d128_window_cap", 1, 16, 16, 512, 512, 128, causal=True, window=100, softcap=30.0,
         seed=52),
    Case("split_nqb2_g8_d128", 1, 32, 4, 256, 300, 128, causal=True, seed=53),
    Case("split_multitoken_g4_lq16_d64", 1, 8, 2, 16, 2000, 64, causal=True, seed=54),
    Case("split_multitoken_g8_lq4_cap", 2, 16, 2, 4, 3000, 128, causal=True, softcap=20.0, seed=55),
    Case("split_multitoken_g2_lq24_d96", 1, 4, 2, 24, 1100, 96, causal=True, window=400, seed=56),
    # prefill kernel (256-row workgroups), full parity
    Case("prefill_big_g16_d128", 1, 256, 16, 256, 256, 128, causal=True, window=90, seed=57),
    Case("prefill_big_g16_d96_noncausal", 1, 256, 16, 256, 200, 96, seed=58),
    # head sizes between the common ones: padded Q.K^T (to 64/96/128) and
    # P.V (to 64/80/128) widths on both kernels
    Case("prefill_big_g16_d112_window_cap", 1, 256, 16, 256, 256, 112, causal=True, window=60, softcap=25.0,
         seed=59),
    Case("prefill_big_g8_d120_noncausal", 1, 256, 32, 256, 256, 120, seed=60),
    Case("split_d120_g4", 1, 16, 4, 40, 900, 120, causal=True, seed=61),
    Case("decode_d80_g8_cap", 2, 16, 2, 1, 1500, 80, causal=True, softcap=40.0, seed=62),
    Case("split_d40_g5_window", 1, 10, 2, 120, 150, 40, causal=True, window=50, seed=63),
    Case("decode_d104_g12", 1, 24, 2, 1, 700, 104, causal=True, seed=64),
    Case("split_d56_g7_fp16", 1, 14, 2, 50, 400, 56, dtype="fp16", seed=65),
    # one 16-row block per unit with many key splits: two workgroups per key
    # range, each with half of V's columns
    Case("halves_multitoken_g4_lq4_cap", 1, 8, 2, 4, 6000, 128, causal=True, softcap=20.0, seed=66),
    Case("halves_decode_window_edges", 2, 16, 1, 1, 5000, 128, causal=True, window=1536, seed=67),
    Case("halves_decode_fp16_cap", 1, 32, 2, 1, 4100, 128, causal=True, softcap=40.0, dtype="fp16", seed=68),
    # one 16-row block and long key ranges per workgroup: 8 waves over 256-key tiles
    Case("wide_decode_g1_d128", 6, 8, 8, 1, 6000, 128, causal=True, seed=69),
    Case("wide_decode_nosplit_d72", 64, 64, 8, 1, 3000, 72, causal=True, seed=70),
    Case("wide_decode_window_cap_fp16", 8, 64, 8, 1, 9000, 128, causal=True, window=5000, softcap=30.0,
         dtype="fp16", seed=71),
    Case("wide_multitoken_g2_lq8_d64_cap", 8, 16, 8, 8, 5000, 64, causal=True, softcap=15.0, seed=72),
    # head sizes that leave the second column half or the padded tail partly empty
    Case("halves_decode_d120_cap", 1, 16, 1, 1, 5000, 120, causal=True, softcap=25.0, seed=73),
    Case("wide_decode_d104", 8, 32, 8, 1, 5000, 104, causal=True, seed=74),
    Case("wide_decode_d40", 8, 64, 8, 1, 4000, 40, causal=True, window=3000, seed=75),
    # degenerate sizes: one key (the output is that key's value row), one key
    # for many non-causal rows, a window longer than the sequence (no window),
    # the largest group with the smallest head size
    Case("single_key_decode", 1, 4, 1, 1, 1, 128, causal=True, seed=76),
    Case("single_key_noncausal_longq_d8", 2, 2, 2, 40, 1, 8, seed=77),
    Case("window_beyond_length_cap", 1, 8, 2, 60, 90, 64, causal=True, window=100000, softcap=10.0,
         seed=78),
    Case("max_group_d8_decode", 1, 16, 1, 1, 300, 8, causal=True, seed=79),
]

CASES_BY_NAME = {c.name: c for c in CASES}
