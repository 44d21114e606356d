"""ctypes binding of libmgqa.so: the C-ABI entry points of include/mgqa.h under
the same names, argument marshalling only.

torch is imported before the library is opened so that the HIP runtime torch
already loaded (same SONAME) is the one the library binds to.  A missing
library raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first; see module docstring)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmgqa.so")
# The measurement build: the same entry points plus the timeline calls of
# include/mgqa_timeline.h.  Chosen with use_timeline_build() before the first
# call of a process.
TIMELINE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmgqa_timeline.so")

# Error codes (include/mgqa.h)
MGQA_OK = 0
MGQA_ERR_NULL = -1
MGQA_ERR_SHAPE = -2
MGQA_ERR_HEAD_DIM = -3
MGQA_ERR_MASK = -4
MGQA_ERR_SOFTCAP = -5
MGQA_ERR_ALIGN = -6
MGQA_ERR_WORKSPACE = -7
MGQA_ERR_HIP = -8
MGQA_ERR_DTYPE = -9
MGQA_ERR_RANGE = -10
MGQA_ERR_UNSUPPORTED = -11

MGQA_BF16 = 0
MGQA_FP16 = 1
MGQA_F32 = 2

# Every symbol the header declares.
EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_fwd_noalloc", "attn_fwd_cache", "attn_fwd_cache_append",
           "kv_cache_append", "attn_workspace_bytes", "attn_plan", "attn_error_string", "attn_version")

# Extra symbols of the timeline build (include/mgqa_timeline.h).
TIMELINE_EXPORTS = ("attn_timeline_layout", "attn_timeline_clear", "attn_timeline_read")

MGQA_NOALLOC_SCRATCH_BYTES = 8 << 20

_lib = None


class LibraryMissing(RuntimeError):
    pass


def use_timeline_build() -> None:
    """Make this process use libmgqa_timeline.so instead of libmgqa.so.  Only
    before the library is opened: one process uses one build."""
    global LIB_PATH
    if _lib is not None and LIB_PATH != TIMELINE_LIB_PATH:
        raise RuntimeError("libmgqa.so is already open in this process")
    LIB_PATH = TIMELINE_LIB_PATH


def load() -> ctypes.CDLL:
    """Open the library (once) and declare the signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} not found: build it with `python -m masked_gqa_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_fwd_ex.restype = i
    lib.attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_noalloc.restype = i
    lib.attn_fwd_cache.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_fwd_cache.restype = i
    lib.attn_fwd_cache_append.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, i, vp, sz,
                                          vp]
    lib.attn_fwd_cache_append.restype = i
    lib.kv_cache_append.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp]
    lib.kv_cache_append.restype = i
    lib.attn_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.attn_workspace_bytes.restype = sz
    lib.attn_plan.argtypes = [i, i, i, i, i, i, i, i, f, i, ctypes.POINTER(ctypes.c_longlong)]
    lib.attn_plan.restype = i
    lib.attn_error_string.argtypes = [i]
    lib.attn_error_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i
    if LIB_PATH == TIMELINE_LIB_PATH:
        lib.attn_timeline_layout.argtypes = [ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.attn_timeline_layout.restype = i
        lib.attn_timeline_clear.argtypes = [vp]
        lib.attn_timeline_clear.restype = i
        lib.attn_timeline_read.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), sz]
        lib.attn_timeline_read.restype = i
    _lib = lib
    return lib


def error_string(code: int) -> str:
    return load().attn_error_string(code).decode()


def attn_fwd(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, stream) -> int:
    return load().attn_fwd(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, int(causal), int(window),
                           float(softcap), stream)


def attn_fwd_ex(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype,
                workspace, workspace_bytes, stream) -> int:
    return load().attn_fwd_ex(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, int(causal), int(window),
                              float(softcap), int(dtype), workspace, int(workspace_bytes), stream)


def attn_fwd_noalloc(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype, stream) -> int:
    return load().attn_fwd_noalloc(q, k, v, out, B, Hq, Hkv, Lq, Lkv, d, int(causal), int(window),
                                   float(softcap), int(dtype), stream)


def attn_fwd_cache(q, k_cache, v_cache, out, B, Hq, Hkv, Lq, S, length, ring_start, d, causal,
                   window, softcap, dtype, workspace, workspace_bytes, stream) -> int:
    return load().attn_fwd_cache(q, k_cache, v_cache, out, B, Hq, Hkv, Lq, S, length, ring_start, d,
                                 int(causal), int(window), float(softcap), int(dtype), workspace,
                                 int(workspace_bytes), stream)


def attn_fwd_cache_append(q, k_cache, v_cache, new_k, new_v, out, B, Hq, Hkv, Lq, S, position,
                          ring_start, d, causal, window, softcap, dtype, workspace, workspace_bytes,
                          stream) -> int:
    return load().attn_fwd_cache_append(q, k_cache, v_cache, new_k, new_v, out, B, Hq, Hkv, Lq, S,
                                        position, ring_start, d, int(causal), int(window),
                                        float(softcap), int(dtype), workspace, int(workspace_bytes),
                                        stream)


def kv_cache_append(k_cache, v_cache, new_k, new_v, B, S, H, D, L, position, cache_dtype, layout,
                    length_out, stream) -> int:
    return load().kv_cache_append(k_cache, v_cache, new_k, new_v, B, S, H, D, L, position,
                                  int(cache_dtype), int(layout), length_out, stream)


def attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, causal, window) -> int:
    return int(load().attn_workspace_bytes(B, Hq, Hkv, Lq, Lkv, d, int(causal), int(window)))


PLAN_FIELDS = ("path", "workgroups", "rows_per_wg", "nsplit", "keys_per_tile", "d_qk_pad",
               "d_pv_pad", "workspace_bytes", "ncol", "pf_pairs", "pf_ramp", "pf_full")


def attn_plan(B, Hq, Hkv, Lq, Lkv, d, causal, window, softcap, dtype=MGQA_BF16):
    """Returns (code, dict) -- dict is empty when code != 0."""
    info = (ctypes.c_longlong * len(PLAN_FIELDS))()
    rc = load().attn_plan(B, Hq, Hkv, Lq, Lkv, d, int(causal), int(window), float(softcap),
                          int(dtype), info)
    if rc != 0:
        return rc, {}
    return rc, dict(zip(PLAN_FIELDS, list(info)))


def attn_version() -> int:
    return int(load().attn_version())


def attn_timeline_layout():
    """(events per record, records) of the timeline build."""
    ev, mw = ctypes.c_int(), ctypes.c_int()
    rc = load().attn_timeline_layout(ctypes.byref(ev), ctypes.byref(mw))
    if rc != 0:
        raise RuntimeError(f"attn_timeline_layout: {error_string(rc)}")
    return ev.value, mw.value


def attn_timeline_clear(stream) -> int:
    return int(load().attn_timeline_clear(stream))


def attn_timeline_read(host_ptr, words) -> int:
    return int(load().attn_timeline_read(ctypes.cast(host_ptr, ctypes.POINTER(ctypes.c_ulonglong)), words))
