"""Masked grouped-query attention for AMD MI355X (gfx950).

    from masked_gqa_attention_amd import attn, make_attention

The compute runs in libmgqa.so (hand-written HIP kernels, C ABI in
include/mgqa.h).  Importing the package does not open the library; the first
call does, and raises if it was not built.
"""
from .synth import WORKLOADS, Workload  # noqa: F401

__all__ = ["attn", "attn_fwd", "attn_cache", "kv_cache_append", "make_attention", "WORKLOADS",
           "Workload"]


def __getattr__(name):
    if name in ("attn", "attn_fwd", "attn_cache", "kv_cache_append", "make_attention", "MgqaError"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
