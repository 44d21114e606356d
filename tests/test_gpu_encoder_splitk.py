"""Encoder-shaped (short, non-causal) sequences with few heads.

Split-K across workgroups: when the key band is too long for the short-band
kernel (more than 768 keys for a block of 48/G positions) and the blocks of
query rows alone give fewer workgroups than compute units, the plan splits
the key axis across workgroups and the last workgroup of each row block
merges the fp32 partials in split order.  Head size 72, 900-1200 tokens, bf16
and fp16, with and without a two-sided window.

With a band of at most 768 keys (the 729-token SigLIP shape) the same
few-head shapes run on the short-band kernel instead, whose eight waves split
the band among themselves and merge in LDS (measured faster than the split
across workgroups for 1 to 8 heads).

Every element against the float64 oracle, plus two runs compared bit for
bit."""
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

# name, B, H, L, window, dtype, seed, path (1: split across workgroups, 2: short-band)
CASES = [
    ("h4_L1000_bf16", 1, 4, 1000, 0, "bf16", 405, 1),
    ("h2_L900_fp16", 1, 2, 900, 0, "fp16", 406, 1),
    ("h1_L1200_window400", 1, 1, 1200, 400, "bf16", 407, 1),
    ("siglip_h4_bf16", 1, 4, 729, 0, "bf16", 401, 2),
    ("siglip_h2_fp16", 1, 2, 729, 0, "fp16", 402, 2),
    ("siglip_h1_window", 1, 1, 729, 100, "bf16", 403, 2),
    ("b2_h2_L500_window", 2, 2, 500, 64, "bf16", 404, 2),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_encoder_splitk(case):
    from masked_gqa_attention_amd import _lib
    name, B, H, L, window, dtype, seed, path = case
    rc, plan = _lib.attn_plan(B, H, H, L, L, 72, 0, window, 0.0, 0 if dtype == "bf16" else 1)
    assert rc == 0 and plan["path"] == path, plan
    assert (plan["nsplit"] > 1) == (path == 1), plan
    announce(f"encoder few heads {name} path={path} nsplit={plan['nsplit']}")
    q = synth.draw_array(seed, (B, H, L, 72), dtype)
    k = synth.draw_array(seed + 1, (B, H, L, 72), dtype)
    v = synth.draw_array(seed + 2, (B, H, L, 72), dtype)
    got = run(q, k, v, dtype, False, window, 0.0)
    again = run(q, k, v, dtype, False, window, 0.0)
    assert np.array_equal(got, again), "output differs between two runs"
    qf, kf, vf = (synth.storage_to_f64(a, dtype) for a in (q, k, v))
    ref = oracle.attention(qf, kf, vf, False, window, 0.0)
    ok, st = compare(got, ref)
    print(name, plan, st, flush=True)
    assert ok, f"{name}: {st}"
    assert st["nrmse"] < 1e-2, f"{name}: {st}"
