"""Split-K for short non-causal (encoder-shaped) sequences: when the blocks of
query rows alone give fewer workgroups than compute units, the plan also
splits the key axis, and the last workgroup of each row block merges the fp32
partials in split order.  SigLIP-shaped inputs (729 tokens, head size 72) with
fewer heads than the benchmark's 16, in bf16 and fp16, with and without a
two-sided window; every element against the float64 oracle, plus two runs
compared bit for bit."""
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

# name, B, H, L, window, dtype, seed
CASES = [
    ("siglip_h4_bf16", 1, 4, 729, 0, "bf16", 401),
    ("siglip_h2_fp16", 1, 2, 729, 0, "fp16", 402),
    ("siglip_h1_window", 1, 1, 729, 100, "bf16", 403),
    ("b2_h2_L500_window", 2, 2, 500, 64, "bf16", 404),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_encoder_splitk(case):
    from masked_gqa_attention_amd import _lib
    name, B, H, L, window, dtype, seed = case
    rc, plan = _lib.attn_plan(B, H, H, L, L, 72, 0, window, 0.0, 0 if dtype == "bf16" else 1)
    assert rc == 0 and plan["path"] == 1 and plan["nsplit"] > 1, plan
    announce(f"encoder split-K {name} nsplit={plan['nsplit']}")
    q = synth.draw_array(seed, (B, H, L, 72), dtype)
    k = synth.draw_array(seed + 1, (B, H, L, 72), dtype)
    v = synth.draw_array(seed + 2, (B, H, L, 72), dtype)
    got = run(q, k, v, dtype, False, window, 0.0)
    again = run(q, k, v, dtype, False, window, 0.0)
    assert np.array_equal(got, again), "split-K output differs between two runs"
    qf, kf, vf = (synth.storage_to_f64(a, dtype) for a in (q, k, v))
    ref = oracle.attention(qf, kf, vf, False, window, 0.0)
    ok, st = compare(got, ref)
    print(name, plan, st, flush=True)
    assert ok, f"{name}: {st}"
    assert st["nrmse"] < 1e-2, f"{name}: {st}"
