"""The torch-facing binding rejects tensors the library cannot take before
any library call: host (CPU) tensors, whose pointers would reach a kernel,
non-contiguous views, wrong element types and a caller `out` that does not
match q.  Runs without a GPU: every call here must raise ValueError."""
import os

import pytest
import torch

from masked_gqa_attention_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmgqa.so not built (python -m masked_gqa_attention_amd.build)")

from masked_gqa_attention_amd import api  # noqa: E402

B, Hq, Hkv, Lq, Lkv, d = 1, 4, 1, 8, 8, 64


def _qkv(dtype=torch.bfloat16):
    return (torch.zeros(B, Hq, Lq, d, dtype=dtype), torch.zeros(B, Hkv, Lkv, d, dtype=dtype),
            torch.zeros(B, Hkv, Lkv, d, dtype=dtype))


def _noncontig(t):
    return t.transpose(-1, -2).contiguous().transpose(-1, -2)  # same shape, strided


@pytest.mark.parametrize("fn", ["attn", "attn_fwd"])
def test_host_tensors_are_rejected(fn):
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU tensor"):
        if fn == "attn":
            api.attn(q, k, v)
        else:
            api.attn_fwd(q, k, v, torch.empty_like(q))


def test_non_contiguous_host_tensors_are_rejected():
    q, k, v = _qkv()
    for args in ((_noncontig(q), k, v), (q, _noncontig(k), v), (q, k, _noncontig(v))):
        with pytest.raises(ValueError):
            api.attn(*args)


def test_wrong_dtype_is_rejected():
    q, k, v = _qkv(torch.float32)
    with pytest.raises(ValueError):
        api.attn(q, k, v)


def test_cache_entry_points_reject_host_tensors():
    q = torch.zeros(B, Hq, 1, d, dtype=torch.bfloat16)
    kc = torch.zeros(B, Hkv, 16, d, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    nk = torch.zeros(B, Hkv, 1, d, dtype=torch.float32)
    nv = torch.zeros_like(nk)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.attn_cache(q, kc, vc, 8)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.attn_cache(q, kc, vc, 8, out=torch.empty_like(q))
    with pytest.raises(ValueError, match="GPU tensor"):
        api.attn_cache_append(q, kc, vc, nk, nv, 3)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.kv_cache_append(kc, vc, nk, nv, 3)


def test_check_helpers_order():
    """The checks name the failing argument."""
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="^q "):
        api.attn(q, k, v)
    with pytest.raises(ValueError, match="out"):
        api._check_out(torch.zeros(2, dtype=torch.bfloat16), q)
