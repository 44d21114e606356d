"""Oracle: KV-cache update at a position (plain PyTorch CPU ops).

TEST INFRASTRUCTURE ONLY (same rule as the attention oracle).

Definition (TensorTonic, "KV Cache Update at a Position"): key_cache and
value_cache are (B, S, H, D), stored in float32 or bfloat16; new_keys and
new_values are (B, L, H, D) float32.  In every batch row and head, slots
position .. position+L-1 receive the new vectors in order, converted to the
cache dtype; every other slot keeps its contents; length = position + L.
Conversion float32 -> bfloat16 is PyTorch's (round to nearest, ties to even).
"""
from __future__ import annotations

import torch


def kv_cache_update(key_cache: torch.Tensor, value_cache: torch.Tensor, new_keys: torch.Tensor,
                    new_values: torch.Tensor, position: int):
    """Returns (key_cache', value_cache', length) for caches laid out
    (B, S, H, D) and new vectors (B, L, H, D); inputs are not modified."""
    B, S, H, D = key_cache.shape
    L = new_keys.shape[1]
    if value_cache.shape != key_cache.shape or new_values.shape != new_keys.shape:
        raise ValueError("shape mismatch")
    if new_keys.shape[0] != B or new_keys.shape[2:] != (H, D):
        raise ValueError("new vectors must be (B, L, H, D) with the cache's B, H, D")
    if not 0 <= position <= S - L:
        raise ValueError("position must satisfy 0 <= position <= S - L")
    k = key_cache.clone()
    v = value_cache.clone()
    k[:, position:position + L] = new_keys.to(torch.float32).to(k.dtype)
    v[:, position:position + L] = new_values.to(torch.float32).to(v.dtype)
    return k, v, position + L
