"""GPU checks of the KV-cache entry points (C ABI through the binding):

* kv_cache_append against the oracle (TensorTonic "KV Cache Update at a
  Position"): the page's worked examples, then random caches of every storage
  type in both layouts, bit for bit;
* attention over a cache prefix (strided K/V rows) and over a ring buffer:
  bit-identical to the same attention over contiguous keys, and within the
  task page's tolerance of the float64 oracle;
* append followed by decode over the filled prefix;
* the fused step (attn_fwd_cache_append): the same output bits and the same
  cache contents as the update followed by attention over the cache, for the
  one-launch split-KV plans (4- and 8-wave, column halves, several position
  blocks, padded head sizes) and the two-launch prefill plans.
"""
import json
import os

import numpy as np
import pytest

import oracle
from masked_gqa_attention_amd import synth

from .cases import compare

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from .gpu_util import announce, to_device, to_host  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_update_examples.json")
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_append_page_examples(idx):
    from masked_gqa_attention_amd import api
    announce(f"append page example {idx}")
    ex = json.load(open(GOLDEN))["examples"][idx]
    kc = torch.tensor(ex["key_cache"], dtype=torch.float32, device="cuda")
    vc = torch.tensor(ex["value_cache"], dtype=torch.float32, device="cuda")
    nk = torch.tensor(ex["new_keys"], dtype=torch.float32, device="cuda")
    nv = torch.tensor(ex["new_values"], dtype=torch.float32, device="cuda")
    length = torch.zeros((), dtype=torch.int32, device="cuda")
    n = api.kv_cache_append(kc, vc, nk, nv, ex["position"], layout=0, length_out=length)
    torch.cuda.synchronize()
    assert n == ex["length"] and int(length.item()) == ex["length"]
    assert torch.equal(kc.cpu(), torch.tensor(ex["out_key_cache"], dtype=torch.float32))
    assert torch.equal(vc.cpu(), torch.tensor(ex["out_value_cache"], dtype=torch.float32))


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("dt", ["f32", "bf16", "fp16"])
def test_append_random_bitwise(layout, dt):
    from masked_gqa_attention_amd import api
    announce(f"append random layout={layout} dtype={dt}")
    rng = np.random.default_rng(11 + layout)
    B, S, H, D, L, pos = 2, 37, 3, 20, 5, 30
    kc0 = torch.from_numpy(rng.standard_normal((B, S, H, D)).astype(np.float32)).to(TD[dt])
    vc0 = torch.from_numpy(rng.standard_normal((B, S, H, D)).astype(np.float32)).to(TD[dt])
    nk = torch.from_numpy(rng.standard_normal((B, L, H, D)).astype(np.float32))
    nv = torch.from_numpy(rng.standard_normal((B, L, H, D)).astype(np.float32))
    want_k, want_v, want_n = oracle.kv_cache_update(kc0, vc0, nk, nv, pos)
    if layout == 1:  # [B,H,S,D] caches and [B,H,L,D] new vectors
        perm = (0, 2, 1, 3)
        kc = kc0.permute(perm).contiguous().cuda()
        vc = vc0.permute(perm).contiguous().cuda()
        n = api.kv_cache_append(kc, vc, nk.permute(perm).contiguous().cuda(),
                                nv.permute(perm).contiguous().cuda(), pos, layout=1)
        got_k, got_v = kc.cpu().permute(perm), vc.cpu().permute(perm)
    else:
        kc, vc = kc0.cuda(), vc0.cuda()
        n = api.kv_cache_append(kc, vc, nk.cuda(), nv.cuda(), pos, layout=0)
        got_k, got_v = kc.cpu(), vc.cpu()
    torch.cuda.synchronize()
    assert n == want_n
    ib = torch.int32 if dt == "f32" else torch.int16
    assert torch.equal(got_k.contiguous().view(ib), want_k.contiguous().view(ib))
    assert torch.equal(got_v.contiguous().view(ib), want_v.contiguous().view(ib))


def _rand(seed, shape, dtype="bf16", sigma=1.0):
    return synth.draw_array(seed, shape, dtype, sigma)


CACHE_CASES = [
    # name, B, Hq, Hkv, Lq, S, length, d, causal, window, softcap
    ("decode_g4_prefix", 2, 8, 2, 1, 3000, 2500, 128, True, 0, 0.0),
    ("decode_g16_window_cap_prefix", 1, 32, 2, 1, 2048, 1999, 128, True, 700, 30.0),
    ("multitoken_g4_prefix", 1, 8, 2, 3, 1500, 1300, 64, True, 200, 0.0),
    ("prefill_g8_prefix", 1, 16, 2, 200, 640, 333, 128, True, 100, 0.0),
    ("prefill_noncausal_prefix_d72", 1, 4, 4, 90, 300, 250, 72, False, 0, 0.0),
]


@pytest.mark.parametrize("case", CACHE_CASES, ids=lambda c: c[0])
def test_attention_over_cache_prefix(case):
    from masked_gqa_attention_amd import api
    name, B, Hq, Hkv, Lq, S, length, d, causal, W, cap = case
    announce(f"cache prefix {name}")
    q = _rand(300, (B, Hq, Lq, d))
    kc = _rand(301, (B, Hkv, S, d))
    vc = _rand(302, (B, Hkv, S, d))
    tq, tk, tv = (to_device(a, "bf16") for a in (q, kc, vc))
    got = api.attn_cache(tq, tk, tv, length, causal=causal, window=W, softcap=cap)
    ref_dev = api.attn(tq, tk[:, :, :length].contiguous(), tv[:, :, :length].contiguous(),
                       causal=causal, window=W, softcap=cap)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref_dev.view(torch.int16))
    gotf = synth.storage_to_f64(to_host(got, "bf16"), "bf16")
    ref = oracle.attention(synth.storage_to_f64(q, "bf16"),
                           synth.storage_to_f64(np.ascontiguousarray(kc[:, :, :length]), "bf16"),
                           synth.storage_to_f64(np.ascontiguousarray(vc[:, :, :length]), "bf16"),
                           causal, W, cap)
    ok, st = compare(gotf, ref)
    assert ok, st


RING_CASES = [
    # name, B, Hq, Hkv, Lq, S(slots), length, ring_start, window, softcap
    ("ring_full_window", 2, 16, 1, 1, 1024, 1024, 300, 1024, 30.0),
    ("ring_partial_fill", 1, 8, 2, 1, 1024, 700, 900, 0, 0.0),
    ("ring_multitoken", 1, 8, 2, 4, 600, 600, 599, 256, 0.0),
    ("ring_start0", 2, 4, 1, 1, 513, 513, 0, 0, 10.0),
    ("ring_long_window_halves", 1, 16, 1, 1, 4096, 4096, 1000, 3000, 30.0),
    ("ring_wide_many_units", 8, 32, 8, 1, 4096, 4096, 1234, 0, 0.0),
]


@pytest.mark.parametrize("case", RING_CASES, ids=lambda c: c[0])
def test_ring_decode_matches_linear(case):
    from masked_gqa_attention_amd import api
    name, B, Hq, Hkv, Lq, S, length, r0, W, cap = case
    announce(f"ring {name}")
    d = 128
    q = _rand(400, (B, Hq, Lq, d))
    lin_k = _rand(401, (B, Hkv, length, d))  # logical keys 0..length-1
    lin_v = _rand(402, (B, Hkv, length, d))
    ring_k = _rand(403, (B, Hkv, S, d))      # unused slots hold other data
    ring_v = _rand(404, (B, Hkv, S, d))
    slots = (r0 + np.arange(length)) % S
    ring_k[:, :, slots] = lin_k
    ring_v[:, :, slots] = lin_v
    tq = to_device(q, "bf16")
    got = api.attn_cache(tq, to_device(ring_k, "bf16"), to_device(ring_v, "bf16"), length,
                         causal=True, window=W, softcap=cap, ring_start=r0)
    lin = api.attn(tq, to_device(lin_k, "bf16"), to_device(lin_v, "bf16"), causal=True, window=W,
                   softcap=cap)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), lin.view(torch.int16))
    ref = oracle.attention(synth.storage_to_f64(q, "bf16"), synth.storage_to_f64(lin_k, "bf16"),
                           synth.storage_to_f64(lin_v, "bf16"), True, W, cap)
    ok, st = compare(synth.storage_to_f64(to_host(got, "bf16"), "bf16"), ref)
    assert ok, st


def test_append_then_decode():
    """Append L new tokens at `position`, then decode over the filled prefix
    [0, position + L): equal to the oracle on the updated cache."""
    from masked_gqa_attention_amd import api
    announce("append then decode")
    B, Hq, Hkv, S, d, pos, L = 2, 16, 2, 4096, 128, 2999, 1
    rng = np.random.default_rng(9)
    kc = torch.from_numpy(rng.standard_normal((B, Hkv, S, d)).astype(np.float32)).to(torch.bfloat16)
    vc = torch.from_numpy(rng.standard_normal((B, Hkv, S, d)).astype(np.float32)).to(torch.bfloat16)
    nk = torch.from_numpy(rng.standard_normal((B, Hkv, L, d)).astype(np.float32))
    nv = torch.from_numpy(rng.standard_normal((B, Hkv, L, d)).astype(np.float32))
    q = torch.from_numpy(rng.standard_normal((B, Hq, L, d)).astype(np.float32)).to(torch.bfloat16)
    perm = (0, 2, 1, 3)  # oracle works in the page's [B,S,H,D] layout
    want_k, want_v, n = oracle.kv_cache_update(kc.permute(perm), vc.permute(perm), nk.permute(perm),
                                               nv.permute(perm), pos)
    dkc, dvc = kc.cuda(), vc.cuda()
    length = api.kv_cache_append(dkc, dvc, nk.cuda(), nv.cuda(), pos, layout=1)
    assert length == n == pos + L
    out = api.attn_cache(q.cuda(), dkc, dvc, length, causal=True, window=1000, softcap=20.0)
    torch.cuda.synchronize()
    kk = want_k.permute(perm)[:, :, :length].float().double().numpy()
    vv = want_v.permute(perm)[:, :, :length].float().double().numpy()
    ref = oracle.attention(q.float().double().numpy(), kk, vv, True, 1000, 20.0)
    ok, st = compare(out.float().cpu().double().numpy(), ref)
    assert ok, st


FUSED_CASES = [
    # name, B, Hq, Hkv, Lq, S, position, d, causal, window, softcap, dtype
    ("decode_g4", 2, 8, 2, 1, 3000, 2499, 128, True, 0, 0.0, "bf16"),
    ("decode_g16_window_cap_halves", 1, 16, 1, 1, 6000, 4999, 128, True, 1536, 30.0, "bf16"),
    ("decode_wide_g1", 6, 8, 8, 1, 7000, 5999, 128, True, 0, 0.0, "bf16"),
    ("multitoken_g4_tile_edge", 1, 8, 2, 3, 1500, 1278, 128, True, 300, 0.0, "bf16"),
    ("multitoken_position_blocks_d64", 1, 16, 2, 16, 2100, 2000, 64, True, 0, 0.0, "bf16"),
    ("fp16_d72_cap", 1, 6, 2, 2, 900, 700, 72, True, 0, 20.0, "fp16"),
    ("noncausal_window_g2", 1, 4, 2, 4, 800, 500, 128, False, 64, 0.0, "bf16"),
    ("multitoken_halves_position_blocks", 1, 8, 1, 8, 5200, 5000, 128, True, 0, 0.0, "bf16"),
    ("halves_d120_cap", 1, 16, 1, 1, 5100, 5000, 120, True, 0, 25.0, "bf16"),
    ("wide_fp16_window", 8, 64, 8, 1, 9100, 9000, 128, True, 5000, 30.0, "fp16"),
    ("prefill_pipelined", 4, 64, 8, 512, 1024, 400, 128, True, 100, 0.0, "bf16"),
    ("prefill_d64", 4, 32, 16, 512, 1200, 600, 64, True, 0, 0.0, "bf16"),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: c[0])
def test_fused_append_matches_update_then_attention(case):
    from masked_gqa_attention_amd import _lib, api
    name, B, Hq, Hkv, Lq, S, pos, d, causal, W, cap, dt = case
    length = pos + Lq
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, length, d, int(causal), W, cap, 0 if dt == "bf16" else 1)
    assert rc == 0
    announce(f"fused append {name} {plan}")
    q = to_device(_rand(500, (B, Hq, Lq, d), dt), dt)
    kc = to_device(_rand(501, (B, Hkv, S, d), dt), dt)
    vc = to_device(_rand(502, (B, Hkv, S, d), dt), dt)
    # The slots about to be written hold NaN: a read of them before the
    # update would reach the output.
    kc[:, :, pos:length] = float("nan")
    vc[:, :, pos:length] = float("nan")
    rng = np.random.default_rng(503)
    nk = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    nv = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    kc1, vc1, kc2, vc2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    got = api.attn_cache_append(q, kc1, vc1, nk, nv, pos, causal=causal, window=W, softcap=cap)
    assert api.kv_cache_append(kc2, vc2, nk, nv, pos, layout=1) == length
    want = api.attn_cache(q, kc2, vc2, length, causal=causal, window=W, softcap=cap)
    torch.cuda.synchronize()
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "K cache differs"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "V cache differs"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "output differs"
    ref = oracle.attention(synth.storage_to_f64(to_host(q, dt), dt),
                           synth.storage_to_f64(to_host(kc2[:, :, :length].contiguous(), dt), dt),
                           synth.storage_to_f64(to_host(vc2[:, :, :length].contiguous(), dt), dt),
                           causal, W, cap)
    ok, st = compare(synth.storage_to_f64(to_host(got, dt), dt), ref)
    print(name, st, flush=True)
    assert ok, st


FUSED_RING_CASES = [
    # name, B, Hq, Hkv, Lq, S, position, ring_start, window, softcap, dtype
    ("ring_full_wrap_g16_window_cap", 1, 16, 1, 1, 4096, 4095, 1000, 4096, 30.0, "bf16"),
    ("ring_partial_g4", 2, 8, 2, 1, 3000, 1499, 2990, 0, 0.0, "bf16"),
    ("ring_multitoken_new_rows_wrap", 1, 4, 2, 4, 600, 592, 5, 300, 0.0, "bf16"),
    ("ring_halves_fp16", 1, 16, 1, 1, 6000, 5999, 123, 1536, 20.0, "fp16"),
    ("ring_wide_g1", 6, 8, 8, 1, 7000, 6999, 3500, 0, 0.0, "bf16"),
]


@pytest.mark.parametrize("case", FUSED_RING_CASES, ids=lambda c: c[0])
def test_fused_append_on_ring(case):
    """The fused step on a ring buffer: the new rows land in slots
    (ring_start + position + i) mod S, and the output equals the ring
    attention over the cache updated by plain indexing, bit for bit."""
    from masked_gqa_attention_amd import _lib, api
    name, B, Hq, Hkv, Lq, S, pos, r0, W, cap, dt = case
    length = pos + Lq
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, length, 128, 1, W, cap, 0 if dt == "bf16" else 1)
    assert rc == 0 and plan["path"] == 1
    announce(f"fused ring append {name} {plan}")
    d = 128
    q = to_device(_rand(510, (B, Hq, Lq, d), dt), dt)
    kc = to_device(_rand(511, (B, Hkv, S, d), dt), dt)
    vc = to_device(_rand(512, (B, Hkv, S, d), dt), dt)
    slots = torch.tensor([(r0 + pos + i) % S for i in range(Lq)], device="cuda")
    kc[:, :, slots] = float("nan")
    vc[:, :, slots] = float("nan")
    rng = np.random.default_rng(513)
    nk = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    nv = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    kc1, vc1, kc2, vc2 = kc.clone(), vc.clone(), kc.clone(), vc.clone()
    got = api.attn_cache_append(q, kc1, vc1, nk, nv, pos, causal=True, window=W, softcap=cap,
                                ring_start=r0)
    kc2[:, :, slots] = nk.to(kc2.dtype)
    vc2[:, :, slots] = nv.to(vc2.dtype)
    want = api.attn_cache(q, kc2, vc2, length, causal=True, window=W, softcap=cap, ring_start=r0)
    torch.cuda.synchronize()
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16)), "K cache differs"
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16)), "V cache differs"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "output differs"
    logical = [(r0 + j) % S for j in range(length)]
    ref = oracle.attention(synth.storage_to_f64(to_host(q, dt), dt),
                           synth.storage_to_f64(to_host(kc2[:, :, logical].contiguous(), dt), dt),
                           synth.storage_to_f64(to_host(vc2[:, :, logical].contiguous(), dt), dt),
                           True, W, cap)
    ok, st = compare(synth.storage_to_f64(to_host(got, dt), dt), ref)
    print(name, st, flush=True)
    assert ok, st
