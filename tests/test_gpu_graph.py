"""HIP graph capture of the library's calls (C ABI through the binding): a
decode step with key splits (partials, arrival counters, last-arrival merge)
and the fused cache-update step are captured once and replayed several
times, with eager work and synchronisation between replays; every replay
must give the eager result bit for bit.  The calls allocate nothing and queue
no memset (the caller's workspace is zero-filled once, before capture, and
the counters return to zero at the end of every call), which is what makes
them capturable."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from masked_gqa_attention_amd import synth  # noqa: E402

from .gpu_util import announce, to_device  # noqa: E402

CASES = [
    # name, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap
    ("decode_split_g4", 2, 8, 2, 1, 3000, 128, True, 0, 0.0),
    ("decode_halves_window_cap", 1, 16, 1, 1, 5000, 128, True, 1536, 30.0),
    ("multitoken_wide", 6, 8, 8, 2, 6000, 128, True, 0, 0.0),
]


def _replays(g, out, want, n=4):
    for r in range(n):
        torch.ones(1024, device="cuda").mul_(2.0)  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {r} differs"


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_attention_in_a_graph(case):
    from masked_gqa_attention_amd import _lib
    name, B, Hq, Hkv, Lq, Lkv, d, causal, W, cap = case
    announce(f"graph {name}")
    q = to_device(synth.draw_array(600, (B, Hq, Lq, d)), "bf16")
    k = to_device(synth.draw_array(601, (B, Hkv, Lkv, d)), "bf16")
    v = to_device(synth.draw_array(602, (B, Hkv, Lkv, d)), "bf16")
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, int(causal), W)
    assert nbytes > 0
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    want = torch.empty_like(q)
    out = torch.empty_like(q)

    def call(o):
        rc = _lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), B, Hq, Hkv, Lq,
                              Lkv, d, causal, W, cap, _lib.MGQA_BF16, ws.data_ptr(), nbytes,
                              torch.cuda.current_stream().cuda_stream)
        assert rc == 0, _lib.error_string(rc)

    call(want)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    _replays(g, out, want)


def test_fused_cache_step_in_a_graph():
    from masked_gqa_attention_amd import _lib
    announce("graph fused cache step")
    B, Hq, Hkv, Lq, S, pos, d = 2, 16, 2, 1, 4096, 3000, 128
    q = to_device(synth.draw_array(610, (B, Hq, Lq, d)), "bf16")
    kc = to_device(synth.draw_array(611, (B, Hkv, S, d)), "bf16")
    vc = to_device(synth.draw_array(612, (B, Hkv, S, d)), "bf16")
    rng = np.random.default_rng(613)
    nk = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    nv = torch.from_numpy(rng.standard_normal((B, Hkv, Lq, d)).astype(np.float32)).cuda()
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, pos + Lq, d, 1, 0)
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    want = torch.empty_like(q)
    out = torch.empty_like(q)

    def call(o):
        rc = _lib.attn_fwd_cache_append(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), nk.data_ptr(),
                                        nv.data_ptr(), o.data_ptr(), B, Hq, Hkv, Lq, S, pos, -1, d, 1,
                                        0, 0.0, _lib.MGQA_BF16, ws.data_ptr() if nbytes else None,
                                        nbytes, torch.cuda.current_stream().cuda_stream)
        assert rc == 0, _lib.error_string(rc)

    call(want)  # writes the new rows; replays write the same rows again
    torch.cuda.synchronize()
    k_after = kc.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    _replays(g, out, want)
    assert torch.equal(kc.view(torch.int16), k_after.view(torch.int16))


def test_api_attn_two_graphs_replayed_in_reverse_order():
    """Two graphs of one split-decode shape captured through api.attn, each
    with its own workspace (zero-filled before capture), replayed in the
    reverse order of capture with eager work in between: every replay equals
    the eager call bit for bit.  Capturing a call whose plan needs a workspace
    without passing one raises instead of sharing the eager cache."""
    from masked_gqa_attention_amd import api
    announce("graph two captures through api.attn")
    B, Hq, Hkv, Lq, Lkv, d = 2, 8, 2, 1, 3000, 128
    q1 = to_device(synth.draw_array(620, (B, Hq, Lq, d)), "bf16")
    q2 = to_device(synth.draw_array(621, (B, Hq, Lq, d)), "bf16")
    k = to_device(synth.draw_array(622, (B, Hkv, Lkv, d)), "bf16")
    v = to_device(synth.draw_array(623, (B, Hkv, Lkv, d)), "bf16")
    want1 = api.attn(q1, k, v, causal=True)
    want2 = api.attn(q2, k, v, causal=True)
    ws1 = api.workspace_for(q1, Hkv, Lkv, causal=True)
    ws2 = api.workspace_for(q2, Hkv, Lkv, causal=True)
    assert ws1 is not None and ws2 is not None
    out1, out2 = torch.empty_like(q1), torch.empty_like(q2)
    torch.cuda.synchronize()
    g1, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        api.attn(q1, k, v, causal=True, out=out1, workspace=ws1)
    with torch.cuda.graph(g2):
        api.attn(q2, k, v, causal=True, out=out2, workspace=ws2)
    for r in range(3):
        for g, out, want in ((g2, out2, want2), (g1, out1, want1)):
            torch.ones(1024, device="cuda").mul_(2.0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {r} differs"
    x = torch.ones(16, device="cuda")
    g3 = torch.cuda.CUDAGraph()
    with pytest.raises(ValueError, match="workspace"):
        with torch.cuda.graph(g3):
            x.mul_(2.0)
            api.attn(q1, k, v, causal=True)
    torch.cuda.synchronize()
