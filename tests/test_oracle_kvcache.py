"""Pins for the KV-cache update oracle: the three worked examples printed on
the TensorTonic page "KV Cache Update at a Position" (tests/golden), and
invariants the page's definition fixes."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from masked_gqa_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_cache_update_examples.json")


def _t(x):
    return torch.tensor(x, dtype=torch.float32)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_page_examples(idx):
    ex = json.load(open(GOLDEN))["examples"][idx]
    k, v, n = oracle.kv_cache_update(_t(ex["key_cache"]), _t(ex["value_cache"]), _t(ex["new_keys"]),
                                     _t(ex["new_values"]), ex["position"])
    assert n == ex["length"]
    assert torch.equal(k, _t(ex["out_key_cache"]))
    assert torch.equal(v, _t(ex["out_value_cache"]))


def test_untouched_slots_and_bf16_rounding():
    rng = np.random.default_rng(5)
    B, S, H, D, L, pos = 2, 9, 3, 5, 4, 3
    kc = torch.from_numpy(rng.standard_normal((B, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    vc = torch.from_numpy(rng.standard_normal((B, S, H, D)).astype(np.float32)).to(torch.bfloat16)
    nk = rng.standard_normal((B, L, H, D)).astype(np.float32)
    nv = rng.standard_normal((B, L, H, D)).astype(np.float32)
    k, v, n = oracle.kv_cache_update(kc, vc, torch.from_numpy(nk), torch.from_numpy(nv), pos)
    assert n == pos + L and k.dtype == torch.bfloat16 and k.shape == kc.shape
    keep = [s for s in range(S) if not pos <= s < pos + L]
    assert torch.equal(k[:, keep].view(torch.int16), kc[:, keep].view(torch.int16))
    assert torch.equal(v[:, keep].view(torch.int16), vc[:, keep].view(torch.int16))
    # written slots: round-to-nearest-even of the float32 bits, computed independently
    want_k = synth.f32_to_bf16_bits(nk).view(np.int16)
    want_v = synth.f32_to_bf16_bits(nv).view(np.int16)
    assert np.array_equal(k[:, pos:pos + L].view(torch.int16).numpy(), want_k)
    assert np.array_equal(v[:, pos:pos + L].view(torch.int16).numpy(), want_v)


def test_position_bounds():
    kc = torch.zeros(1, 4, 1, 2)
    nk = torch.ones(1, 2, 1, 2)
    for pos in (0, 2):
        k, _, n = oracle.kv_cache_update(kc, kc, nk, nk, pos)
        assert n == pos + 2 and k.sum() == 4
    for pos in (-1, 3):
        with pytest.raises(ValueError):
            oracle.kv_cache_update(kc, kc, nk, nk, pos)
