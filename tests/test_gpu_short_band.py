"""The short-band kernel: workgroups of three 16-row blocks on eight waves,
each wave taking its own contiguous 32-key steps of the block's key band
(bands of at most 768 keys, head sizes 49..96: the 729-token encoder and
shapes like it), a two-pass softmax over the wave's scores, and a merge of
the eight wave states in wave order.  Each case first checks that the plan
takes that path, then compares every element with the float64 oracle and two
runs bit for bit; the cache step on such a plan must equal the update followed
by the attention over the cache.  Bands longer than 768 keys keep the
split-KV kernel (three row blocks on four waves), checked the same way."""
import numpy as np
import pytest

import oracle
from masked_gqa_attention_amd import synth

from .cases import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from .gpu_util import announce, run, to_device, to_host  # noqa: E402

# name, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype, seed
CASES = [
    ("encoder_bf16", 1, 16, 16, 729, 729, 72, False, 0, 0.0, "bf16", 601),
    ("encoder_fp16", 1, 16, 16, 729, 729, 72, False, 0, 0.0, "fp16", 602),
    ("d96_causal_softcap_fp16", 1, 16, 16, 729, 729, 96, True, 0, 30.0, "fp16", 603),
    ("d64_two_sided_window", 2, 8, 8, 729, 729, 64, False, 200, 0.0, "bf16", 604),
    # band of 300 keys: ten 32-key steps, two per wave, the last three waves idle
    ("idle_waves_d72", 2, 16, 16, 400, 300, 72, False, 0, 0.0, "bf16", 605),
    # two heads per kv head (rows are (position, head) pairs), causal window, softcap
    ("g2_causal_window_cap_d80", 1, 16, 8, 800, 800, 80, True, 300, 30.0, "bf16", 606),
    # five heads per kv head: 9 positions, 45 of the 48 rows used
    ("g5_causal_d96_fp16", 1, 20, 4, 600, 600, 96, True, 0, 0.0, "fp16", 607),
    # bottom-right alignment with Lq < Lkv, band start not a multiple of 32
    ("bottom_right_window_d72", 2, 16, 16, 400, 533, 72, True, 77, 12.0, "fp16", 608),
]

# Three row blocks over bands longer than 768 keys (or head size 48): the
# split-KV kernel on four waves.
SPLIT_CASES = [
    ("g3_d48_window_bottom_right", 1, 3, 1, 4096, 4500, 48, True, 1000, 0.0, "bf16", 615),
    ("g3_d48_window_softcap_fp16", 1, 3, 1, 4096, 4500, 48, True, 1000, 20.0, "fp16", 616),
    ("long_band_d72", 1, 16, 16, 729, 1500, 72, True, 0, 0.0, "bf16", 617),
]


def _plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dt, path=2):
    from masked_gqa_attention_amd import _lib
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, d, int(causal), window, softcap, 0 if dt == "bf16" else 1)
    assert rc == 0
    assert plan["path"] == path and plan["rows_per_wg"] == 48, plan
    assert plan["nsplit"] == 1, plan
    if path == 2:
        assert plan["keys_per_tile"] == 96 and plan["workspace_bytes"] == 0, plan
    return plan


def _check(name, B, Hq, Hkv, Lq, Lkv, d, causal, window, cap, dt, seed):
    q = synth.draw_array(seed, (B, Hq, Lq, d), dt)
    k = synth.draw_array(seed + 1000, (B, Hkv, Lkv, d), dt)
    v = synth.draw_array(seed + 2000, (B, Hkv, Lkv, d), dt)
    got = run(q, k, v, dt, causal, window, cap)
    again = run(q, k, v, dt, causal, window, cap)
    assert np.array_equal(got, again), "output differs between two runs"
    ref = oracle.attention(*(synth.storage_to_f64(a, dt) for a in (q, k, v)), causal, window, cap)
    ok, st = compare(got, ref)
    print(name, st, flush=True)
    assert ok, f"{name}: {st}"


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_short_band(case):
    plan = _plan(*case[1:11])
    announce(f"short band {case[0]} {plan}")
    _check(*case)


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: c[0])
def test_three_blocks_long_band(case):
    plan = _plan(*case[1:11], path=1)
    assert plan["keys_per_tile"] == 128, plan
    announce(f"three row blocks, long band {case[0]} {plan}")
    _check(*case)


def test_short_band_cache_step():
    from masked_gqa_attention_amd import api
    B, Hq, Hkv, Lq, S, pos, d, dt = 32, 32, 8, 12, 800, 688, 64, "bf16"
    length = pos + Lq
    plan = _plan(B, Hq, Hkv, Lq, length, d, True, 0, 0.0, dt)
    announce(f"short band cache step {plan}")
    q = to_device(synth.draw_array(611, (B, Hq, Lq, d), dt), dt)
    kc = to_device(synth.draw_array(612, (B, Hkv, S, d), dt), dt)
    vc = to_device(synth.draw_array(613, (B, Hkv, S, d), dt), dt)
    kc[:, :, pos:length] = float("nan")  # a read of a slot before its update would reach the output
    vc[:, :, pos:length] = float("nan")
    rng = np.random.default_rng(614)
    nk = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    nv = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    kc1, vc1, kc2, vc2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    got = api.attn_cache_append(q, kc1, vc1, nk, nv, pos, causal=True)
    assert api.kv_cache_append(kc2, vc2, nk, nv, pos, layout=1) == length
    want = api.attn_cache(q, kc2, vc2, length, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "K cache differs"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "V cache differs"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "output differs"
    ref = oracle.attention(synth.storage_to_f64(to_host(q, dt), dt),
                           synth.storage_to_f64(to_host(kc2[:, :, :length].contiguous(), dt), dt),
                           synth.storage_to_f64(to_host(vc2[:, :, :length].contiguous(), dt), dt),
                           True, 0, 0.0)
    ok, st = compare(synth.storage_to_f64(to_host(got, dt), dt), ref)
    print("fused", st, flush=True)
    assert ok, st


# Hot queries (scores spread over tens of units): on the split-KV kernel the
# running maximum grows tile after tile, so the rescale of the accumulators
# (one wave-uniform branch for all row blocks, rows that need none multiplied
# by exactly 1) is taken often; on the short-band kernel the scores of a wave
# span a wide range below its single maximum.
# name, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype, qscale, rows, keys_per_tile, path
HOT_CASES = [
    ("hot_short_band", 1, 16, 16, 729, 729, 72, False, 0, 0.0, "fp16", 6.0, 48, 96, 2),
    ("hot_short_band_cap", 1, 16, 16, 729, 729, 72, False, 0, 30.0, "bf16", 12.0, 48, 96, 2),
    ("hot_short_band_190", 5, 16, 16, 190, 190, 72, False, 0, 0.0, "bf16", 12.0, 48, 96, 2),
    ("hot_3blocks_long_band", 1, 16, 16, 729, 1500, 72, True, 0, 0.0, "bf16", 12.0, 48, 128, 1),
    ("hot_2blocks_long_band", 1, 16, 16, 700, 900, 80, True, 0, 0.0, "bf16", 12.0, 32, 128, 1),
    ("hot_4blocks_g3", 1, 48, 16, 729, 729, 40, True, 0, 0.0, "fp16", 5.0, 64, 128, 1),
]


@pytest.mark.parametrize("case", HOT_CASES, ids=lambda c: c[0])
def test_hot_queries_on_row_blocks(case):
    from masked_gqa_attention_amd import _lib
    name, B, Hq, Hkv, Lq, Lkv, d, causal, window, cap, dt, qscale, rows, kpt, path = case
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, d, int(causal), window, cap, 0 if dt == "bf16" else 1)
    assert rc == 0 and plan["path"] == path and plan["rows_per_wg"] == rows and plan["keys_per_tile"] == kpt, plan
    announce(f"hot row blocks {name} {plan}")
    seed = 700 + len(name)
    q = synth.draw_array(seed, (B, Hq, Lq, d), dt)
    q = synth.f32_to_storage((synth.storage_to_f64(q, dt) * qscale).astype(np.float32), dt)
    k = synth.draw_array(seed + 1, (B, Hkv, Lkv, d), dt)
    v = synth.draw_array(seed + 2, (B, Hkv, Lkv, d), dt)
    got = run(q, k, v, dt, causal, window, cap)
    again = run(q, k, v, dt, causal, window, cap)
    assert np.array_equal(got, again), "output differs between two runs"
    ref = oracle.attention(*(synth.storage_to_f64(a, dt) for a in (q, k, v)), causal, window, cap)
    ok, st = compare(got, ref)
    print(name, st, flush=True)
    assert ok, f"{name}: {st}"
