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


# One zero-initialised workspace per (device, stream) for eager calls.  The
# library leaves the arrival counters at zero after every completed call, so a
# workspace is cleared only when it is first allocated or grown.
_ws_lock = threading.Lock()
_ws_cache: dict = {}


def _check_gpu(name: str, t: torch.Tensor, dtypes, device: torch.device | None = None) -> None:
    """A contiguous GPU tensor of one of `dtypes` (on `device` if given)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {sorted(map(str, dtypes))}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_out(out: torch.Tensor, like: torch.Tensor) -> None:
    _check_gpu("out", out, (like.dtype,), like.device)
    if tuple(out.shape) != tuple(like.shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(like.shape)}")


def workspace_for(q: torch.Tensor, Hkv: int, Lkv: int, causal: bool = False, window: int = 0) -> torch.Tensor | None:
    """A new zero-filled workspace for attention of q [B,Hq,Lq,d] over Lkv keys
    of Hkv kv heads (None when the plan needs none).  For callers that capture
    the call into a graph: fill it before capture and give every graph its own."""
    B, Hq, Lq, d = q.shape
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, causal, window)
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=q.device)


def _workspace(nbytes: int, device: torch.device, stream_ptr: int,
               given: torch.Tensor | None) -> torch.Tensor | None:
    if given is not None:
        _check_gpu("workspace", given, (torch.uint8,), device)
        if given.numel() < nbytes:
            raise ValueError(f"workspace holds {given.numel()} bytes, the plan needs {nbytes}")
        return given
    if nbytes == 0:
        return None
    if torch.cuda.is_current_stream_capturing():
        # A graph replays its kernels with the addresses it captured; a shared
        # cached workspace would be used by several graphs (and zeroed only by
        # whichever captured its allocation), so graphs bring their own.
        raise ValueError("this shape needs a workspace: inside graph capture pass workspace= "
                         "(api.workspace_for(...), zero-filled before capture, one per graph)")
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
         window: int = 0, softcap: float = 0.0, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Masked GQA attention forward on the GPU.  q [B,Hq,Lq,d], k/v [B,Hkv,Lkv,d],
    contiguous bf16 or fp16 device tensors of one dtype.  Returns out [B,Hq,Lq,d].
    workspace: optional uint8 device tensor (workspace_for); required inside
    graph capture when the plan needs one."""
    _check_gpu("q", q, tuple(_DTYPES))
    _check_gpu("k", k, (q.dtype,), q.device)
    _check_gpu("v", v, (q.dtype,), q.device)
    B, Hq, Hkv, Lq, Lkv, d = _shape(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, causal, window)
    ws = _workspace(nbytes, q.device, stream, workspace)
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
    _check_gpu("q", q, (torch.bfloat16,))
    _check_gpu("k", k, (torch.bfloat16,), q.device)
    _check_gpu("v", v, (torch.bfloat16,), q.device)
    B, Hq, Hkv, Lq, Lkv, d = _shape(q, k, v)
    _check_out(out, q)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, stream)
    if rc != 0:
        raise MgqaError(rc, "attn_fwd")


_CACHE_DTYPES = {torch.bfloat16: _lib.MGQA_BF16, torch.float16: _lib.MGQA_FP16,
                 torch.float32: _lib.MGQA_F32}


def kv_cache_append(k_cache: torch.Tensor, v_cache: torch.Tensor, new_k: torch.Tensor,
                    new_v: torch.Tensor, position: int, layout: int = 1,
                    length_out: torch.Tensor | None = None) -> int:
    """Write L new float32 key/value vectors into the caches at `position`
    (in place) and return position + L.  layout 1: caches [B,H,S,D], new
    [B,H,L,D] (what attn_cache reads); layout 0: caches [B,S,H,D], new
    [B,L,H,D].  If length_out (int32 device scalar) is given, the kernel writes
    position + L into it as well."""
    _check_gpu("k_cache", k_cache, tuple(_CACHE_DTYPES))
    _check_gpu("v_cache", v_cache, (k_cache.dtype,), k_cache.device)
    _check_gpu("new_k", new_k, (torch.float32,), k_cache.device)
    _check_gpu("new_v", new_v, (torch.float32,), k_cache.device)
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape or new_k.shape != new_v.shape:
        raise ValueError("caches and new vectors must be 4-D, pairwise of one shape")
    if layout == 1:
        B, H, S, D = k_cache.shape
        L = new_k.shape[2]
        ok = new_k.shape == (B, H, L, D)
    else:
        B, S, H, D = k_cache.shape
        L = new_k.shape[1]
        ok = new_k.shape == (B, L, H, D)
    if not ok:
        raise ValueError("new vectors do not match the cache shape for this layout")
    if length_out is not None:
        _check_gpu("length_out", length_out, (torch.int32,), k_cache.device)
        if length_out.numel() < 1:
            raise ValueError("length_out must hold at least one int32")
    stream = torch.cuda.current_stream(k_cache.device).cuda_stream
    rc = _lib.kv_cache_append(k_cache.data_ptr(), v_cache.data_ptr(), new_k.data_ptr(),
                              new_v.data_ptr(), B, S, H, D, L, position, _CACHE_DTYPES[k_cache.dtype],
                              layout, length_out.data_ptr() if length_out is not None else None,
                              stream)
    if rc != 0:
        raise MgqaError(rc, "kv_cache_append")
    return position + L


def attn_cache(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, length: int,
               causal: bool = False, window: int = 0, softcap: float = 0.0, ring_start: int = -1,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Attention of q [B,Hq,Lq,d] over the first `length` keys of caches
    [B,Hkv,S,d] (ring_start = -1), or over a ring buffer whose logical key j is
    slot (ring_start + j) % S."""
    _check_gpu("q", q, tuple(_DTYPES))
    _check_gpu("k_cache", k_cache, (q.dtype,), q.device)
    _check_gpu("v_cache", v_cache, (q.dtype,), q.device)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q and the caches must be 4-D: [B,Hq,Lq,d], [B,Hkv,S,d]")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, S, dk = k_cache.shape
    if Bk != B or dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape mismatch")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, length, d, causal, window)
    ws = _workspace(nbytes, q.device, stream, workspace)
    rc = _lib.attn_fwd_cache(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(),
                             B, Hq, Hkv, Lq, S, length, ring_start, d, causal, window, softcap,
                             _DTYPES[q.dtype], ws.data_ptr() if ws is not None else None, nbytes,
                             stream)
    if rc != 0:
        raise MgqaError(rc, "attn_fwd_cache")
    return out


def attn_cache_append(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      new_k: torch.Tensor, new_v: torch.Tensor, position: int, causal: bool = True,
                      window: int = 0, softcap: float = 0.0, ring_start: int = -1,
                      out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One step over a cache: write the Lq new float32 key/value rows
    new_k, new_v [B,Hkv,Lq,d] as logical keys position .. position+Lq-1 of
    the caches [B,Hkv,S,d] (in place, rounded to the cache dtype; slot j, or
    (ring_start + j) % S for a ring), then attend with q [B,Hq,Lq,d] (rows at
    positions position .. position+Lq-1) over logical keys 0 .. position+Lq-1.
    For a linear cache, the same result as kv_cache_append followed by
    attn_cache; on the decode path it is a single kernel launch."""
    _check_gpu("q", q, tuple(_DTYPES))
    _check_gpu("k_cache", k_cache, (q.dtype,), q.device)
    _check_gpu("v_cache", v_cache, (q.dtype,), q.device)
    _check_gpu("new_k", new_k, (torch.float32,), q.device)
    _check_gpu("new_v", new_v, (torch.float32,), q.device)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q and the caches must be 4-D: [B,Hq,Lq,d], [B,Hkv,S,d]")
    B, Hq, Lq, d = q.shape
    Bk, Hkv, S, dk = k_cache.shape
    if Bk != B or dk != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape mismatch")
    if new_k.shape != (B, Hkv, Lq, d) or new_v.shape != new_k.shape:
        raise ValueError("new rows must be [B, Hkv, Lq, d]")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    nbytes = _lib.attn_workspace_bytes(B, Hq, Hkv, Lq, position + Lq, d, causal, window)
    ws = _workspace(nbytes, q.device, stream, workspace)
    rc = _lib.attn_fwd_cache_append(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    new_k.data_ptr(), new_v.data_ptr(), out.data_ptr(), B, Hq, Hkv,
                                    Lq, S, position, ring_start, d, causal, window, softcap,
                                    _DTYPES[q.dtype],
                                    ws.data_ptr() if ws is not None else None, nbytes, stream)
    if rc != 0:
        raise MgqaError(rc, "attn_fwd_cache_append")
    return out


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
