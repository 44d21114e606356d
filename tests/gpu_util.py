"""Helpers for the GPU tests: move storage arrays to the device and back, and
run the library through its Python binding (which calls the C ABI)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from masked_gqa_attention_amd import api, synth

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16}


def to_device(arr: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run(q, k, v, dtype, causal, window, softcap) -> np.ndarray:
    """GPU attention on storage arrays; returns the output as float64."""
    tq, tk, tv = (to_device(a, dtype) for a in (q, k, v))
    out = api.attn(tq, tk, tv, causal=causal, window=window, softcap=softcap)
    torch.cuda.synchronize()
    return synth.storage_to_f64(to_host(out, dtype), dtype)


def announce(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
