"""attn_fwd_noalloc, the entry point that allocates nothing (its split
partials and counters live in a device array inside the library), called
through the C ABI: its output equals attn_fwd_ex's with a caller workspace bit
for bit, and is within the tolerance of the float64 oracle, on two calls in a
row -- the second with a smaller input and a different split plan -- and again
on the first shape (the scratch keeps the last call's contents; the counters
must be back at zero), plus a prefill-path shape that needs no scratch."""
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

# name, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, seed
SHAPES = [
    ("long_window_decode_halves", 2, 32, 2, 1, 9000, 128, True, 4096, 30.0, 801),
    ("small_split_decode", 1, 8, 2, 1, 3000, 128, True, 0, 0.0, 802),
    ("multitoken_d64", 2, 16, 4, 4, 2500, 64, True, 0, 0.0, 803),
]


def _call(fn_name, tq, tk, tv, out, shape, ws=None):
    from masked_gqa_attention_amd import _lib
    _, B, Hq, Hkv, Lq, Lkv, d, causal, window, cap, _ = shape
    stream = torch.cuda.current_stream().cuda_stream
    if fn_name == "ex":
        nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, causal, window)
        rc = _lib.attn_fwd_ex(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), B, Hq, Hkv, Lq, Lkv,
                              d, causal, window, cap, _lib.MGQA_BF16, ws.data_ptr() if nbytes else None, nbytes,
                              stream)
    else:
        rc = _lib.attn_fwd_noalloc(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), out.data_ptr(), B, Hq, Hkv, Lq,
                                   Lkv, d, causal, window, cap, _lib.MGQA_BF16, stream)
    assert rc == 0, _lib.error_string(rc)


def _run_pair(shape):
    from masked_gqa_attention_amd import _lib
    name, B, Hq, Hkv, Lq, Lkv, d, causal, window, cap, seed = shape
    rc, plan = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, cap)
    assert rc == 0
    announce(f"noalloc {name} {plan}")
    q = synth.draw_array(seed, (B, Hq, Lq, d))
    k = synth.draw_array(seed + 1, (B, Hkv, Lkv, d))
    v = synth.draw_array(seed + 2, (B, Hkv, Lkv, d))
    tq, tk, tv = (to_device(a, "bf16") for a in (q, k, v))
    ws = torch.zeros(max(plan["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
    want, got = torch.empty_like(tq), torch.empty_like(tq)
    _call("ex", tq, tk, tv, want, shape, ws)
    _call("noalloc", tq, tk, tv, got, shape)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{name}: differs from attn_fwd_ex"
    ref = oracle.attention(*(synth.storage_to_f64(a, "bf16") for a in (q, k, v)), causal, window, cap)
    ok, st = compare(synth.storage_to_f64(to_host(got, "bf16"), "bf16"), ref)
    print(name, st, flush=True)
    assert ok, f"{name}: {st}"
    return plan


def test_noalloc_matches_attn_fwd_ex_on_consecutive_calls():
    big = _run_pair(SHAPES[0])
    small = _run_pair(SHAPES[1])
    assert big["nsplit"] > 1 and small["nsplit"] > 1
    assert small["workspace_bytes"] < big["workspace_bytes"]
    _run_pair(SHAPES[2])
    _run_pair(SHAPES[0])  # the first shape again, after the others used the scratch


def test_noalloc_prefill_path_needs_no_scratch():
    _run_pair(("prefill_no_scratch", 1, 16, 2, 300, 300, 128, True, 100, 20.0, 804))
