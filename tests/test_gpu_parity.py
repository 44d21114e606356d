"""GPU parity: the HIP path against the float64 oracle, element by element, on
seeded inputs, through the C ABI (Python binding).  Tolerance rtol = atol =
2e-2 as stated on the task page ("Hard Constraints"), plus a normalised RMS
error bound of 1e-2 as a tighter sanity check on the bulk of the output.
"""
import numpy as np
import pytest

import oracle
from masked_gqa_attention_amd import synth

from .cases import CASES, as_f64, compare, make_inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from .gpu_util import announce, run  # noqa: E402


def _band_edges(i, Lq, Lkv, causal, W):
    pos = Lkv - Lq + i
    lo, hi = 0, Lkv - 1
    if causal:
        hi = min(hi, pos)
    if W > 0:
        lo = max(lo, pos - W + 1)
        if not causal:
            hi = min(hi, pos + W - 1)
    return lo, hi


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_parity_case(case):
    announce(case.name)
    q, k, v = make_inputs(case)
    qf, kf, vf = as_f64(case, (q, k, v))
    ref = oracle.attention(qf, kf, vf, case.causal, case.window, case.softcap)
    got = run(q, k, v, case.dtype, case.causal, case.window, case.softcap)
    ok, st = compare(got, ref)
    assert ok, f"{case.name}: {st}"
    assert st["nrmse"] < 1e-2, f"{case.name}: {st}"
    if case.kind == "onehot":
        # Exactly zero off the band, 1/n_i (rounded to the storage type) on it.
        for b in range(case.B):
            for h in range(case.Hq):
                for i in range(case.Lq):
                    lo, hi = _band_edges(i, case.Lq, case.Lkv, case.causal, case.window)
                    row = got[b, h, i]
                    assert np.all(row[:lo] == 0.0) and np.all(row[hi + 1:] == 0.0)
                    want = synth.storage_to_f64(synth.f32_to_storage(
                        np.array([1.0 / (hi - lo + 1)], np.float32), case.dtype), case.dtype)[0]
                    assert np.all(row[lo:hi + 1] == want), (b, h, i, row[lo:hi + 1], want)
    if case.kind == "const":
        assert np.all(got == 0.8125)
    if case.kind == "hot" and case.softcap > 0:
        # The softcap must matter for this input, so parity here proves it is applied.
        nocap = oracle.attention(qf, kf, vf, case.causal, case.window, 0.0)
        assert not compare(nocap, ref)[0]


def test_determinism_bitwise():
    import torch as T
    from masked_gqa_attention_amd import api
    from .cases import CASES_BY_NAME
    from .gpu_util import to_device
    # one case per kernel form: split (several row blocks, fp16), split with
    # column halves, wide split, register-staged prefill, pipelined prefill
    for name in ("prefill_window_cap_g8", "decode_g16_window_cap", "decode_g4_kv3000", "split_nqb3_d72_fp16",
                 "halves_decode_fp16_cap", "wide_decode_g1_d128", "prefill_big_g16_d96_noncausal",
                 "prefill_big_g16_d128"):
        c = CASES_BY_NAME[name]
        announce(f"determinism {name}")
        q, k, v = (to_device(a, c.dtype) for a in make_inputs(c))
        outs = [api.attn(q, k, v, c.causal, c.window, c.softcap).clone() for _ in range(4)]
        T.cuda.synchronize()
        for o in outs[1:]:
            assert T.equal(o.view(T.int16), outs[0].view(T.int16))


def test_attn_fwd_self_allocating_matches_ex():
    """attn_fwd (library-allocated workspace) gives the same bits as
    attn_fwd_ex with a caller workspace, on a split-decode shape."""
    import torch as T
    from masked_gqa_attention_amd import api
    from .cases import CASES_BY_NAME
    from .gpu_util import to_device
    for name in ("decode_g4_kv3000", "prefill_causal_g4_L200"):
        c = CASES_BY_NAME[name]
        announce(f"attn_fwd {name}")
        q, k, v = (to_device(a, c.dtype) for a in make_inputs(c))
        a = api.attn(q, k, v, c.causal, c.window, c.softcap)
        b = T.empty_like(q)
        api.attn_fwd(q, k, v, b, c.causal, c.window, c.softcap)
        T.cuda.synchronize()
        assert T.equal(a.view(T.int16), b.view(T.int16))


def test_workspace_reuse_across_shapes():
    """One workspace serves calls of different shapes in turn without being
    cleared: a split decode with a large partial region, then shapes with many
    row blocks and key splits (more arrival counters), then the decode again.
    Each result must equal, bit for bit, the same call on a fresh zero-filled
    workspace."""
    import torch as T
    from masked_gqa_attention_amd import _lib
    from .cases import CASES_BY_NAME
    from .gpu_util import to_device
    names = ["decode_g4_kv3000", "prefill_causal_g8_bottomright", "split_multitoken_g8_lq4_cap",
             "decode_g4_kv3000", "prefill_causal_g8_bottomright"]
    sizes = []
    for name in set(names):
        c = CASES_BY_NAME[name]
        sizes.append(_lib.attn_workspace_bytes(c.B, c.Hq, c.Hkv, c.Lq, c.Lkv, c.d, c.causal, c.window))
    shared = T.zeros(max(sizes), dtype=T.uint8, device="cuda")
    stream = T.cuda.current_stream().cuda_stream

    def call(c, tensors, ws):
        q, k, v = tensors
        out = T.empty_like(q)
        nbytes = _lib.attn_workspace_bytes(c.B, c.Hq, c.Hkv, c.Lq, c.Lkv, c.d, c.causal, c.window)
        assert nbytes > 0
        rc = _lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), c.B, c.Hq,
                              c.Hkv, c.Lq, c.Lkv, c.d, c.causal, c.window, c.softcap,
                              _lib.MGQA_BF16, ws.data_ptr(), ws.numel(), stream)
        assert rc == 0, _lib.error_string(rc)
        return out

    for name in names:
        c = CASES_BY_NAME[name]
        announce(f"workspace reuse {name}")
        tensors = [to_device(a, c.dtype) for a in make_inputs(c)]
        got = call(c, tensors, shared)
        fresh = call(c, tensors, T.zeros(max(sizes), dtype=T.uint8, device="cuda"))
        T.cuda.synchronize()
        assert T.equal(got.view(T.int16), fresh.view(T.int16)), name


def test_suffix_consistency_decode_vs_prefill():
    """Bottom-right alignment across the two kernels: decode of the last
    query row equals the last row of a full prefill, and a 4-row chunk equals
    the last 4 rows."""
    from .cases import Case
    for causal, W, cap in [(True, 0, 0.0), (True, 300, 30.0), (False, 0, 0.0)]:
        c = Case("suffix", 1, 8, 2, 700, 700, 128, causal=causal, window=W, softcap=cap, seed=77)
        announce(f"suffix causal={causal} W={W} cap={cap}")
        q, k, v = make_inputs(c)
        full = run(q, k, v, c.dtype, causal, W, cap)
        for lq in (1, 2, 4):
            part = run(np.ascontiguousarray(q[:, :, -lq:]), k, v, c.dtype, causal, W, cap)
            ok, st = compare(part, full[:, :, -lq:], rtol=1e-2, atol=1e-2)
            assert ok, (lq, st)


def test_gqa_equals_repeated_kv_on_gpu():
    from .cases import Case
    c = Case("gqa", 1, 16, 2, 150, 150, 128, causal=True, window=40, softcap=10.0, seed=78)
    announce("gqa vs mha")
    q, k, v = make_inputs(c)
    a = run(q, k, v, c.dtype, c.causal, c.window, c.softcap)
    kr = np.ascontiguousarray(np.repeat(k, 8, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, 8, axis=1))
    b = run(q, kr, vr, c.dtype, c.causal, c.window, c.softcap)
    ok, st = compare(a, b, rtol=1e-2, atol=1e-2)
    assert ok, st


def test_python_errors():
    import torch as T
    from masked_gqa_attention_amd import api
    q = T.zeros(1, 4, 8, 100, dtype=T.bfloat16, device="cuda")
    k = T.zeros(1, 1, 8, 100, dtype=T.bfloat16, device="cuda")
    with pytest.raises(api.MgqaError) as e:
        api.attn(q, k, k)
    assert e.value.code == -3
    q = T.zeros(1, 4, 9, 64, dtype=T.bfloat16, device="cuda")
    k = T.zeros(1, 1, 8, 64, dtype=T.bfloat16, device="cuda")
    with pytest.raises(api.MgqaError) as e:
        api.attn(q, k, k, causal=True)
    assert e.value.code == -4
