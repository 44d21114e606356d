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

Every case asserts that the plan takes the prefill path with head size 128,
and compares sampled rows (all band edges plus seeded random rows) element
by element; the smaller ones are compared in full.
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


def _rows(B, Hq, Lq, Lkv, window, seed, n_random=160):
    rng = np.random.default_rng(seed)
    off = Lkv - Lq
    edges = {0, 1, 31, 32, 33, 63, 64, Lq // 2, Lq - 33, Lq - 32, Lq - 2, Lq - 1}
    if window > 0:
        for w in (window - 1, window, window + 1):
            edges.update({w - off - 1, w - off, w - off + 1, w - 1, w})
    rows = set()
    for i in edges:
        if 0 <= i < Lq:
            for b in range(B):
                rows.update({(b, 0, i), (b, Hq - 1, i), (b, int(rng.integers(Hq)), i)})
    while len(rows) < 3 * B * len(edges) + n_random:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Lq))))
    return sorted(rows)


def _inputs(name, B, Hq, Hkv, Lq, Lkv, dtype, qscale, seed):
    q = synth.draw_array(seed, (B, Hq, Lq, 128), dtype)
    k = synth.draw_array(seed + 1, (B, Hkv, Lkv, 128), dtype)
    v = synth.draw_array(seed + 2, (B, Hkv, Lkv, 128), dtype)
    qf = synth.storage_to_f64(q, dtype) * qscale
    if name.startswith("fixref_cap50"):
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
def test_prefill128_parity(case):
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
    if B * Hq * Lq * Lkv <= 24 * 1024 * 1024:
        ref = oracle.attention(qf, kf, vf, causal, window, softcap)
        ok, st = compare(got, ref)
    else:
        rows = _rows(B, Hq, Lq, Lkv, window, seed)
        ref = oracle.attention_rows(qf, kf, vf, rows, causal, window, softcap)
        ok, st = compare(np.stack([got[b, h, i] for (b, h, i) in rows]), ref)
    print(name, st, flush=True)
    assert ok, f"{name}: {st}"
    assert st["nrmse"] < 1e-2, f"{name}: {st}"
    if name.startswith("fixref_cap50"):
        # The constructed batch really sits at the lower bound: its scaled
        # scores are all below -c/2 before the softcap.
        G = Hq // Hkv
        s = np.stack([qf[1, h, :64] @ kf[1, h // G].T for h in range(0, Hq, 4)]) / np.sqrt(128)
        assert s.max() < -softcap / 2
