"""Seeded random sweep of shapes through every plan the library can pick
(pipelined prefill with its work-item layouts, generic prefill, 4- and 8-wave
split-KV with one to four row blocks, key splits, column halves, the
short-band kernel): GQA ratios 1 to 16, head sizes that are
multiples of 8 up to 128, ragged query and key lengths, bottom-right causal
masks, one- and two-sided windows, softcaps, bf16 and fp16.  Every element is
compared with the float64 oracle within the task page's tolerance, and two
runs must agree bit for bit.  The shapes come from a fixed generator seed, so
the sweep is the same on every run; sizes keep the oracle within seconds."""
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

N_CASES = 48
MAX_PAIRS = 6_000_000   # Hq * Lq * Lkv per batch row, bounds the oracle's cost


def _shapes():
    rng = np.random.default_rng(20261203)
    out = []
    while len(out) < N_CASES:
        G = int(rng.choice([1, 2, 3, 4, 8, 16]))
        Hkv = int(rng.integers(1, 5))
        d = 8 * int(rng.integers(1, 17))
        kind = rng.integers(0, 4)  # 0 decode-like, 1 short prefill, 2 long band, 3 many heads
        if kind == 3:
            Hkv = int(rng.choice([8, 16]))
            G = int(rng.choice([2, 4, 8]))
            Lkv = int(rng.integers(150, 600))
            Lq = int(rng.integers(Lkv // 2, Lkv + 1))
        elif kind == 0:
            Lq = int(rng.integers(1, 9))
            Lkv = int(rng.integers(Lq, 6000))
        elif kind == 1:
            Lkv = int(rng.integers(2, 900))
            Lq = int(rng.integers(1, Lkv + 1))
        else:
            Lkv = int(rng.integers(500, 3000))
            Lq = int(rng.integers(Lkv // 2, Lkv + 1))
        B = int(rng.integers(1, 3)) if kind != 3 else 2
        causal = bool(rng.integers(0, 2))
        window = int(rng.choice([0, 0, 1, 7, 64, 300, 5000]))
        softcap = float(rng.choice([0.0, 0.0, 15.0, 50.0, 70.0]))
        dtype = "bf16" if rng.integers(0, 3) else "fp16"
        if (causal or window > 0) and Lq > Lkv:
            continue
        if G * Hkv * Lq * Lkv > MAX_PAIRS:
            continue
        out.append((len(out), B, G * Hkv, Hkv, Lq, Lkv, d, causal, window, softcap, dtype))
    return out


def _targeted():
    """Random lengths and options on shapes built to land on the plans a
    small random shape rarely reaches: the pipelined head-size-128 prefill,
    the generic prefill (two and one 16-row blocks per wave), 8-wave split-KV
    with one and with three row blocks, and column halves."""
    rng = np.random.default_rng(20261204)
    rng_wide = np.random.default_rng(20261205)
    out = []
    for r in range(2):
        L = int(rng.integers(200, 400))
        out.append(("pipe", 2, 64, 8, L, L + int(rng.integers(0, 50)), 128, True,
                    int(rng.choice([0, 37, 150])), float(rng.choice([0.0, 40.0])), ["bf16", "fp16"][r]))
        L = int(rng.integers(520, 640))
        out.append(("prefill", 2, 64, 16, L, L, int(rng.choice([48, 64, 96])), bool(r), 0,
                    float(rng.choice([0.0, 25.0])), "bf16"))
        out.append(("wide_decode", 32, 8 * int(rng.choice([1, 2, 4])), 8, 1, int(rng.integers(1100, 2000)),
                    8 * int(rng.integers(4, 17)), True, int(rng.choice([0, 900])), 0.0, ["bf16", "fp16"][r]))
        L = int(rng.integers(600, 760))
        out.append(("wide_rows", 1, 16, 16, L, L, 8 * int(rng.integers(5, 13)), False,
                    int(rng.choice([0, 150])), float(rng.choice([0.0, 30.0])), ["fp16", "bf16"][r]))
        out.append(("halves", 1, 16, 1, int(rng.integers(1, 3)), int(rng.integers(5000, 9000)), 128, True,
                    int(rng.integers(2000, 4000)), float(rng.choice([0.0, 30.0])), "bf16"))
        # Head-size-128 prefill work items: causal ramp pairs, and half blocks.
        L = int(rng.integers(262, 290))
        out.append(("items_pairs", 2, 64, 8, L, L, 128, True, 0, float(rng.choice([0.0, 45.0])),
                    ["bf16", "fp16"][r]))
        L = int(rng.integers(340, 356))
        out.append(("items_halves", 3, 32, 8, L, L, 128, False, 0, float(rng.choice([0.0, 20.0])),
                    ["fp16", "bf16"][r]))
        # Few heads over a short band: the short-band kernel with few workgroups.
        out.append(("few_heads", 1, 2, 2, int(rng.integers(600, 729)), 729, 72, False,
                    int(rng.choice([0, 200])), 0.0, ["fp16", "bf16"][r]))
        # Generic prefill at head sizes 104-120 (one 16-row block per wave).
        L = int(rng_wide.integers(520, 640))
        out.append(("prefill_one_block", 2, 64, 16, L, L + int(rng_wide.integers(0, 40)),
                    int(rng_wide.choice([104, 112, 120])), bool(1 - r), int(rng_wide.choice([0, 190])),
                    float(rng_wide.choice([0.0, 35.0])), ["fp16", "bf16"][r]))
    return [(N_CASES + i,) + t[1:] for i, t in enumerate(out)]


SHAPES = _shapes() + _targeted()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"s{s[0]}")
def test_random_shape(shape):
    from masked_gqa_attention_amd import _lib
    i, B, Hq, Hkv, Lq, Lkv, d, causal, window, cap, dt = shape
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, d, int(causal), window, cap, 0 if dt == "bf16" else 1)
    assert rc == 0, (shape, rc)
    announce(f"sweep {shape} plan={plan}")
    seed = 7000 + 10 * i
    q = synth.draw_array(seed, (B, Hq, Lq, d), dt)
    k = synth.draw_array(seed + 1, (B, Hkv, Lkv, d), dt)
    v = synth.draw_array(seed + 2, (B, Hkv, Lkv, d), dt)
    got = run(q, k, v, dt, causal, window, cap)
    again = run(q, k, v, dt, causal, window, cap)
    assert np.array_equal(got, again), f"{shape}: two runs differ"
    ref = oracle.attention(*(synth.storage_to_f64(a, dt) for a in (q, k, v)), causal, window, cap)
    ok, st = compare(got, ref)
    print(shape, plan, st, flush=True)
    assert ok, f"{shape}: {st}"
