"""Parity at the largest K/V unit the library accepts (2^30 elements per
(batch row, kv head), 2 GiB of bf16 per K or V tensor) on the generic prefill
kernel: head size 112 (one 16-row block per wave) and head size 64 (two),
each sweeping the whole band of about 9.6M / 16.8M keys under a causal mask,
so that the kernel's 32-bit offsets reach their top end and the last tile is
ragged (2^30 / 112 keys is no multiple of the 64-key tile).

Input recipe as for the head-size-128 case: one seeded block of 2^17 keys,
copy t rotated by t times a fixed odd stride (different for K and V, so no
two copies pair the same keys with the same values); the oracle sees the
full tensors in float64 and computes a few sampled rows over the whole band."""
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

BLOCK = 1 << 17


def _long_sequence(seed: int, stride: int, n: int, d: int) -> np.ndarray:
    blk = synth.draw_array(seed, (BLOCK, d), "bf16")
    out = np.empty((n, d), np.uint16)
    for t in range(-(-n // BLOCK)):
        lo, hi = t * BLOCK, min(n, (t + 1) * BLOCK)
        out[lo:hi] = np.roll(blk, stride * t, axis=0)[:hi - lo]
    return out


CASES = [
    # name, d, Hq (one kv head), Lq, rows per workgroup expected
    ("generic_one_block_d112_g16", 112, 16, 2048, 128),
    ("generic_two_blocks_d64_g16", 64, 16, 4096, 256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_largest_unit_generic_prefill(case):
    from masked_gqa_attention_amd import _lib, api
    name, d, Hq, Lq, rows_wg = case
    n = (1 << 30) // d
    rc, plan = _lib.attn_plan(1, Hq, 1, Lq, n, d, 1, 0, 0.0)
    assert rc == 0 and plan["path"] == 0 and plan["rows_per_wg"] == rows_wg, plan
    assert _lib.attn_plan(1, Hq, 1, Lq, n + 1, d, 1, 0, 0.0)[0] == _lib.MGQA_ERR_RANGE
    announce(f"max size {name} keys={n} {plan}")
    k = _long_sequence(841 + d, 7919, n, d)[None, None]
    v = _long_sequence(842 + d, 104729, n, d)[None, None]
    q = synth.draw_array(843 + d, (1, Hq, Lq, d), "bf16")
    dk, dv = to_device(k, "bf16"), to_device(v, "bf16")
    out = api.attn(to_device(q, "bf16"), dk, dv, causal=True)
    torch.cuda.synchronize()
    got = synth.storage_to_f64(to_host(out, "bf16"), "bf16")
    del dk, dv, out
    torch.cuda.empty_cache()
    assert np.isfinite(got).all()
    rng = np.random.default_rng(850 + d)
    rows = {(0, h, i) for h in (0, Hq - 1) for i in {0, Lq // 2, Lq - 1}}
    while len(rows) < 12:
        rows.add((0, int(rng.integers(Hq)), int(rng.integers(Lq))))
    rows = sorted(rows)
    kf, vf = synth.storage_to_f64(k, "bf16"), synth.storage_to_f64(v, "bf16")
    ref = oracle.attention_rows(synth.storage_to_f64(q, "bf16"), kf, vf, rows, True, 0, 0.0)
    ok, st = compare(np.stack([got[r] for r in rows]), ref)
    print(name, st, flush=True)
    assert ok, f"{name}: {st}"
    assert st["nrmse"] < 1e-2, f"{name}: {st}"
