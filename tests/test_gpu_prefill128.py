"""Parity of the head-size-128 prefill kernel (the software-pipelined one)
against the float64 oracle, on shapes chosen to reach each of its paths:

* the fixed softmax reference used under a softcap with bf16 (c <= 57.5),
  including rows whose every visible score sits at the softcap's lower bound
  -c, where the probabilities are the smallest the fixed reference produces;
* the running-maximum path just above that softcap threshold, with a large
  softcap, with fp16, and without a softcap;
* GQA groups that do not divide the 128-row workgroup (rows left unused),
  ragged lengths that are not multiples of the 32-key tile, bottom-right
  causal alignment with Lq < Lkv, a non-causal (two-sided) window.

Every case asserts that the plan takes the prefill path with head size 128
and compares every output element with the float64 oracle (run head by head
in a process pool for the larger shapes).

ITEM_CASES reach each work-item layout of the kernel -- ramp blocks paired
(with an odd ramp's middle block alone), half blocks of 64 rows (one 16-row
block per wave) for every group size that allows them, a partial last block
kept whole beside halved ones -- on the fixed-reference and running-maximum
paths and with fp16; each asserts the layout it is meant to reach.

The anti-aligned batches ("fixref_cap50_hot", "fixref_cap57p5_floor") push
every visible score to the softcap's lower bound -c.  At c = 57.5, the largest
softcap that keeps the fixed reference, the smallest probability is about
2^-126, so its products with values below 1 sit below the float32 normal
range inside the P.V products; the case shows the output still matches.
"""
import numpy as np
import pytest

import oracle
from masked_gqa_attention_amd import synth

from .cases import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from .gpu_util import announce, run  # noqa: E402

# name, B, Hq, Hkv, Lq, Lkv, causal, window, softcap, dtype, q scale, seed
CASES = [
    ("fixref_cap50_hot", 2, 16, 2, 1024, 1024, True, 300, 50.0, "bf16", 12.0, 301),
    ("fixref_cap57p5_floor", 2, 16, 2, 1024, 1024, True, 300, 57.5, "bf16", 12.0, 311),
    ("fixref_cap57p5_floor_short_rows", 2, 64, 8, 300, 300, True, 0, 57.5, "bf16", 12.0, 312),
    ("fixref_cap57_ragged", 2, 32, 4, 777, 1061, True, 0, 57.0, "bf16", 8.0, 302),
    ("runmax_cap58", 2, 32, 4, 777, 1061, True, 0, 58.0, "bf16", 8.0, 303),
    ("runmax_cap500_window", 2, 16, 2, 1040, 1040, True, 129, 500.0, "bf16", 30.0, 304),
    ("runmax_fp16_cap", 2, 16, 2, 1024, 1024, True, 200, 20.0, "fp16", 4.0, 305),
    ("nocap_g3_rows_unused", 2, 24, 8, 700, 700, True, 0, 0.0, "bf16", 1.0, 306),
    ("nocap_g5_bottom_right", 2, 20, 4, 900, 1500, True, 0, 0.0, "bf16", 1.0, 307),
    ("fixref_g7_two_sided_window", 2, 28, 4, 640, 640, False, 90, 30.0, "bf16", 6.0, 308),
    ("nocap_g16_long_window", 1, 64, 4, 512, 2080, True, 513, 0.0, "bf16", 1.0, 309),
    ("nocap_g1_noncausal", 4, 16, 16, 520, 520, False, 0, 0.0, "bf16", 1.0, 310),
]

# name, B, Hq, Hkv, Lq, Lkv, causal, window, softcap, dtype, q scale, seed, layout
# layout: "pairs", "odd" (pairs and one middle block alone), "halves",
# "all_halves", "mixed" (pairs, whole and half blocks)
ITEM_CASES = [
    ("items_odd_ramp_fixref", 2, 32, 4, 660, 700, True, 0, 50.0, "bf16", 8.0, 320, "odd"),
    ("items_mixed_window_g2", 2, 32, 16, 1280, 1280, True, 256, 0.0, "bf16", 1.0, 321, "mixed"),
    ("items_mixed_partial_last_g4", 2, 64, 16, 1003, 1003, True, 0, 30.0, "bf16", 6.0, 322, "mixed"),
    ("items_halves_partial_last_g4", 1, 64, 16, 977, 977, True, 0, 0.0, "bf16", 1.0, 323, "halves"),
    ("items_all_halves_g1_fixref", 2, 16, 16, 1280, 1280, True, 0, 30.0, "bf16", 6.0, 324, "all_halves"),
    ("items_all_halves_g2_fp16", 2, 32, 16, 640, 640, True, 0, 20.0, "fp16", 4.0, 325, "all_halves"),
    ("items_all_halves_g8_fixref", 2, 32, 4, 640, 640, True, 0, 50.0, "bf16", 8.0, 326, "all_halves"),
]


def _inputs(name, B, Hq, Hkv, Lq, Lkv, dtype, qscale, seed):
    q = synth.draw_array(seed, (B, Hq, Lq, 128), dtype)
    k = synth.draw_array(seed + 1, (B, Hkv, Lkv, 128), dtype)
    v = synth.draw_array(seed + 2, (B, Hkv, Lkv, 128), dtype)
    qf = synth.storage_to_f64(q, dtype) * qscale
    if "_floor" in name or name.startswith("fixref_cap50"):
        # Batch 1: every query anti-aligned with every key, so each visible
        # score is pushed to the softcap's lower bound.
        kf = synth.storage_to_f64(k, dtype)
        u = kf[1].mean(axis=1, keepdims=True)                         # [Hkv,1,d]
        u = u / np.linalg.norm(u, axis=-1, keepdims=True)
        kf[1] = kf[1] * 0.05 + 4.0 * u                               # keys ~ +u
        G = Hq // Hkv
        qf[1] = -400.0 * np.repeat(u, G, axis=0) + 0.01 * qf[1]      # queries ~ -u
        k = synth.f32_to_storage(kf.astype(np.float32), dtype)
    q = synth.f32_to_storage(qf.astype(np.float32), dtype)
    return q, k, v


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_prefill128_parity(case, oracle_pool):
    _check_case(case, oracle_pool)


@pytest.mark.parametrize("case", ITEM_CASES, ids=lambda c: c[0])
def test_prefill128_item_layouts(case, oracle_pool):
    from masked_gqa_attention_amd import _lib
    name, B, Hq, Hkv, Lq, Lkv, causal, window, softcap, dtype, qscale, seed, layout = case
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, 128, int(causal), window, softcap,
                              0 if dtype == "bf16" else 1)
    assert rc == 0 and plan["path"] == 0, plan
    items = plan["workgroups"] // (B * Hkv)
    pairs, ramp, full = plan["pf_pairs"], plan["pf_ramp"], plan["pf_full"]
    halves = items - pairs - full
    got = {"pairs": pairs > 0 and halves == 0 and ramp % 2 == 0,
           "odd": pairs > 0 and ramp % 2 == 1,
           "halves": pairs == 0 and full > 0 and halves > 0,
           "all_halves": pairs == 0 and full == 0 and halves > 0,
           "mixed": pairs > 0 and full > 0 and halves > 0}[layout]
    assert got, (layout, plan)
    _check_case(case[:-1], oracle_pool)


def _check_case(case, oracle_pool):
    from masked_gqa_attention_amd import _lib
    name, B, Hq, Hkv, Lq, Lkv, causal, window, softcap, dtype, qscale, seed = case
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, 128, int(causal), window, softcap,
                              0 if dtype == "bf16" else 1)
    assert rc == 0 and plan["path"] == 0 and plan["d_qk_pad"] == 128, plan
    announce(f"prefill128 {name}")
    q, k, v = _inputs(name, B, Hq, Hkv, Lq, Lkv, dtype, qscale, seed)
    got = run(q, k, v, dtype, causal, window, softcap)
    assert np.isfinite(got).all()
    qf, kf, vf = (synth.storage_to_f64(a, dtype) for a in (q, k, v))
    ref = oracle_pool.attention(qf, kf, vf, causal, window, softcap)
    ok, st = compare(got, ref)
    print(name, st, f"{got.size} elements compared", flush=True)
    assert ok, f"{name}: {st}"
    assert st["nrmse"] < 1e-2, f"{name}: {st}"
    if "_floor" in name or name.startswith("fixref_cap50"):
        # The constructed batch really sits at the lower bound: its scaled
        # scores are all below -c/2 before the softcap.
        G = Hq // Hkv
        s = np.stack([qf[1, h, :64] @ kf[1, h // G].T for h in range(0, Hq, 4)]) / np.sqrt(128)
        assert s.max() < -softcap / 2
