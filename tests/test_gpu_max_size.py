"""Parity at the largest K/V unit the library accepts: one (batch row, kv
head) of 2^30 elements, 2 GiB of bf16 per K or V tensor.  At this size the
kernels' 32-bit byte offsets and descriptor ranges reach their limit (2^31
bytes), so these cases check the address arithmetic of every path at its top
end: a split decode over 8M keys, the pipelined prefill kernel and the
split-KV kernel sweeping the whole 8M-key band of their rows, and cache
decodes (linear and ring) whose unused slots hold NaN, which must never be
read.

Input recipe: drawing 2^30 normal values per tensor takes too long for a test,
so a long K (V) is built from one seeded block of 2^17 keys, copy t rotated
by t times a fixed odd stride, with different strides for K and V so that no
two copies pair the same keys with the same values.  Any misplaced tile read
therefore changes the result.  The oracle sees the full tensors (float64, a
few rows at a time)."""
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

D = 128
N_MAX = (1 << 30) // D          # keys in the largest unit at d = 128
BLOCK = 1 << 17


def _long_sequence(seed: int, stride: int) -> np.ndarray:
    blk = synth.draw_array(seed, (BLOCK, D), "bf16")
    out = np.empty((N_MAX, D), np.uint16)
    for t in range(N_MAX // BLOCK):
        out[t * BLOCK:(t + 1) * BLOCK] = np.roll(blk, stride * t, axis=0)
    return out


@pytest.fixture(scope="module")
def long_kv():
    announce(f"building K/V of {N_MAX} keys x {D}")
    k = _long_sequence(801, 7919)[None, None]
    v = _long_sequence(802, 104729)[None, None]
    dk, dv = to_device(k, "bf16"), to_device(v, "bf16")
    kf, vf = synth.storage_to_f64(k, "bf16"), synth.storage_to_f64(v, "bf16")
    yield dk, dv, kf, vf
    del dk, dv
    torch.cuda.empty_cache()


MAX_CASES = [
    # name, Hq, Lq, causal, query scale, expected path (0 prefill, 1 split), key splits > 1
    ("decode_g8_full_band", 8, 1, False, 4.0, 1, True),
    ("prefill_pipelined_causal_g16", 16, 2048, True, 1.0, 0, False),
    ("split_kernel_unsplit_causal_g16", 16, 1024, True, 1.0, 1, False),
]


@pytest.mark.parametrize("case", MAX_CASES, ids=lambda c: c[0])
def test_largest_unit(case, long_kv):
    from masked_gqa_attention_amd import _lib, api
    name, Hq, Lq, causal, qscale, path, split = case
    rc, plan = _lib.attn_plan(1, Hq, 1, Lq, N_MAX, D, int(causal), 0, 0.0)
    assert rc == 0 and plan["path"] == path and (plan["nsplit"] > 1) == split, plan
    announce(f"max size {name} {plan}")
    dk, dv, kf, vf = long_kv
    q = synth.draw_array(810 + Lq, (1, Hq, Lq, D), "bf16")
    if qscale != 1.0:
        q = synth.f32_to_storage((synth.storage_to_f64(q, "bf16") * qscale).astype(np.float32), "bf16")
    out = api.attn(to_device(q, "bf16"), dk, dv, causal=causal)
    torch.cuda.synchronize()
    got = synth.storage_to_f64(to_host(out, "bf16"), "bf16")
    assert np.isfinite(got).all()
    rng = np.random.default_rng(820 + Lq)
    rows = {(0, h, i) for h in (0, Hq - 1) for i in {0, Lq // 2, Lq - 1}}
    while len(rows) < min(12, Hq * Lq):
        rows.add((0, int(rng.integers(Hq)), int(rng.integers(Lq))))
    rows = sorted(rows)
    ref = oracle.attention_rows(synth.storage_to_f64(q, "bf16"), kf, vf, rows, causal, 0, 0.0)
    ok, st = compare(np.stack([got[r] for r in rows]), ref)
    print(name, st, flush=True)
    assert ok, f"{name}: {st}"
    assert st["nrmse"] < 1e-2, f"{name}: {st}"


RING_CASES = [
    # d, ring_start (-1: linear cache)
    (128, -1), (128, 0), (120, -1), (120, 0), (120, "wrap"),
]


@pytest.mark.parametrize("d,r0", RING_CASES, ids=lambda x: str(x))
def test_largest_cache_never_reads_unused_slots(d, r0):
    """Decode over a cache of S = 2^30/d slots (the largest accepted) holding
    `length` keys; every other slot is NaN.  Window W: the row sees the last W
    logical keys only, and since the mask depends on the distance p - j alone,
    the oracle over the last T >= W logical keys gives the same rows.  Only those
    T keys hold random data; the other filled slots hold zeros."""
    from masked_gqa_attention_amd import api
    S = (1 << 30) // d
    length, W, T, cap, Hq = S // 2 + 77, 1000, 4096, 30.0, 4
    ring = -1 if r0 == -1 else (0 if r0 == 0 else S - 5)
    announce(f"max cache d={d} ring_start={ring} S={S} length={length}")
    dev = "cuda:0"
    logical = torch.arange(length, device=dev, dtype=torch.int64)
    slots = logical if ring < 0 else (ring + logical) % S
    tail = slots[length - T:]
    q = synth.draw_array(830 + d, (1, Hq, 1, d), "bf16")
    kt = synth.draw_array(831 + d, (1, 1, T, d), "bf16")
    vt = synth.draw_array(832 + d, (1, 1, T, d), "bf16")
    caches = []
    for data in (kt, vt):
        c = torch.full((1, 1, S, d), float("nan"), dtype=torch.bfloat16, device=dev)
        c[0, 0, slots] = 0
        c[0, 0, tail] = to_device(data, "bf16")[0, 0]
        caches.append(c)
    out = api.attn_cache(to_device(q, "bf16"), caches[0], caches[1], length, causal=True,
                         window=W, softcap=cap, ring_start=ring)
    torch.cuda.synchronize()
    got = synth.storage_to_f64(to_host(out, "bf16"), "bf16")
    del caches
    torch.cuda.empty_cache()
    ref = oracle.attention(synth.storage_to_f64(q, "bf16"), synth.storage_to_f64(kt, "bf16"),
                           synth.storage_to_f64(vt, "bf16"), True, W, cap)
    ok, st = compare(got, ref)
    print(d, ring, st, flush=True)
    assert ok, st
