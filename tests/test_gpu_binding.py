"""The torch-facing binding on the GPU: tensors the library cannot take --
non-contiguous views, float32, a host tensor mixed with device tensors, an
`out` of the wrong shape or dtype, a too-small workspace -- raise ValueError
before any library call; valid calls through every entry point run."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from masked_gqa_attention_amd import api, synth  # noqa: E402

from .gpu_util import announce, to_device  # noqa: E402


def _qkv(Lq=4, Lkv=300):
    q = to_device(synth.draw_array(900, (1, 8, Lq, 128)), "bf16")
    k = to_device(synth.draw_array(901, (1, 2, Lkv, 128)), "bf16")
    v = to_device(synth.draw_array(902, (1, 2, Lkv, 128)), "bf16")
    return q, k, v


def test_rejections_before_any_library_call():
    announce("binding rejections")
    q, k, v = _qkv()
    strided = k.transpose(-1, -2).contiguous().transpose(-1, -2)
    with pytest.raises(ValueError, match="contiguous"):
        api.attn(q, strided, v)
    with pytest.raises(ValueError, match="dtype"):
        api.attn(q.float(), k.float(), v.float())
    with pytest.raises(ValueError, match="on cpu|GPU tensor"):
        api.attn(q, k.cpu(), v)
    with pytest.raises(ValueError, match="shape"):
        api.attn(q, k, v, out=torch.empty(1, 8, 3, 128, dtype=q.dtype, device=q.device))
    with pytest.raises(ValueError, match="dtype"):
        api.attn(q, k, v, out=torch.empty_like(q, dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        api.attn_fwd(q, k, v, torch.empty(1, 8, 4, 64, dtype=q.dtype, device=q.device))
    with pytest.raises(ValueError, match="contiguous"):
        api.attn_fwd(q, strided, v, torch.empty_like(q))
    kc = torch.zeros(1, 2, 512, 128, dtype=q.dtype, device=q.device)
    vc = torch.zeros_like(kc)
    nk = torch.zeros(1, 2, 4, 128, dtype=torch.float32, device=q.device)
    with pytest.raises(ValueError, match="shape"):
        api.attn_cache(q, kc, vc, 300, out=torch.empty(1, 8, 4, 120, dtype=q.dtype, device=q.device))
    with pytest.raises(ValueError, match="on cpu|GPU tensor"):
        api.attn_cache_append(q, kc, vc, nk.cpu(), nk, 100)
    with pytest.raises(ValueError, match="dtype"):
        api.attn_cache_append(q, kc, vc, nk.half(), nk, 100)
    with pytest.raises(ValueError, match="workspace"):
        api.attn(q, k, v, causal=True, workspace=torch.zeros(8, dtype=torch.uint8, device=q.device))
    torch.cuda.synchronize()


def test_valid_calls_with_caller_out_and_workspace():
    announce("binding valid calls")
    q, k, v = _qkv(Lq=1, Lkv=3000)
    want = api.attn(q, k, v, causal=True)
    out = torch.empty_like(q)
    ws = api.workspace_for(q, 2, 3000, causal=True)
    got = api.attn(q, k, v, causal=True, out=out, workspace=ws)
    assert got is out
    out2 = torch.empty_like(q)
    api.attn_fwd(q, k, v, out2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), want.view(torch.int16))
