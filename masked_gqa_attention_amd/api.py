"""Torch-facing wrapper over the C ABI: checks tensors, takes their device
pointers and torch's current stream, and calls attn_fwd_ex.  Every step of
the attention itself runs in the HIP kernels of libmgqa.so; torch provides
device memory and the stream only.

The call shape mirrors the task page "TPU v6e Masked GQA Kernel Optimization"
("What You Submit": make_attention(cfg) returns f(q, k, v); bf16 in and out,
output in q's shape).
"""
from __future__ import annotations

import threading

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.MGQA_BF16, torch.float16: _lib.MGQA_FP16}


class MgqaError(ValueError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {_lib.error_string(code)} (code {code})")


# One zero-initialised workspace per (device, stream).  The library leaves the
# arrival counters at zero after every completed call, so a workspace is
# cleared only when it is first allocated or grown.
_ws_lock = threading.Lock()
_ws_cache: dict = {}


def _workspace(nbytes: int, device: torch.device, stream_ptr: int) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    key = (device.index, stream_ptr)
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


def _shape(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D: [B,Hq,Lq,d], [B,Hkv,Lkv,d], [B,Hkv,Lkv,d]")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, Lkv, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return B, Hq, Hkv, Lq, Lkv, d


def attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
         window: int = 0, softcap: float = 0.0, out: torch.Tensor | None = None) -> torch.Tensor:
    """Masked GQA attention forward on the GPU.  q [B,Hq,Lq,d], k/v [B,Hkv,Lkv,d],
    contiguous bf16 or fp16 device tensors of one dtype.  Returns out [B,Hq,Lq,d]."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dtype not in _DTYPES or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, bfloat16 or float16")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    B, Hq, Hkv, Lq, Lkv, d = _shape(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, causal, window)
    ws = _workspace(nbytes, q.device, stream)
    rc = _lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, _DTYPES[q.dtype],
                          ws.data_ptr() if ws is not None else None, nbytes, stream)
    if rc != 0:
        raise MgqaError(rc, "attn_fwd_ex")
    return out


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
             causal: bool = False, window: int = 0, softcap: float = 0.0) -> None:
    """The bf16 entry point attn_fwd exactly as the C ABI has it (the library
    allocates its own stream-ordered workspace)."""
    B, Hq, Hkv, Lq, Lkv, d = _shape(q, k, v)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, stream)
    if rc != 0:
        raise MgqaError(rc, "attn_fwd")


def make_attention(cfg: dict):
    """cfg keys: batch, q_len, kv_len, num_q_heads, num_kv_heads, head_dim,
    causal, window, softcap (seed and name are accepted and ignored: the
    kernels never branch on them).  Returns f(q, k, v) -> out."""
    causal = bool(cfg.get("causal", False))
    window = int(cfg.get("window") or 0)
    softcap = float(cfg.get("softcap") or 0.0)
    expect = (cfg.get("batch"), cfg.get("num_q_heads"), cfg.get("q_len"), cfg.get("head_dim"))

    def f(q, k, v):
        if all(x is not None for x in expect) and tuple(q.shape) != tuple(expect):
            raise ValueError(f"q shape {tuple(q.shape)} does not match cfg {expect}")
        return attn(q, k, v, causal=causal, window=window, softcap=softcap)

    return f
