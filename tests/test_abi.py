"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, rejects bad arguments before any HIP call, and plans the expected
path for each workload.  No compute call is made here (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from masked_gqa_attention_amd import _lib
from masked_gqa_attention_amd.synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgqa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libmgqa.so not built (python -m masked_gqa_attention_amd.build)")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*([a-z_]+)\s*\(", text, flags=re.M)))


def test_header_matches_binding_list():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_header_symbol():
    lib = _lib.load()
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in header_functions():
        assert name in exported, name


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


@pytest.mark.skipif(not os.path.exists(_lib.TIMELINE_LIB_PATH), reason="libmgqa_timeline.so not built")
def test_timeline_build_exports():
    """The measurement build exports every entry point of both headers; the
    library proper has none of the timeline calls."""
    tl_header = os.path.join(ROOT, "include", "mgqa_timeline.h")
    assert header_functions(tl_header) == sorted(_lib.TIMELINE_EXPORTS)
    tl = _exported(_lib.TIMELINE_LIB_PATH)
    for name in header_functions() + header_functions(tl_header):
        assert name in tl, name
    plain = _exported(_lib.LIB_PATH)
    assert not plain & set(_lib.TIMELINE_EXPORTS)


@pytest.mark.skipif(not os.path.exists(_lib.TIMELINE_LIB_PATH), reason="libmgqa_timeline.so not built")
def test_timeline_calls_validate_before_hip():
    """Layout, and the argument checks of the read call, need no GPU."""
    tl = ctypes.CDLL(_lib.TIMELINE_LIB_PATH)
    ev, mw = ctypes.c_int(), ctypes.c_int()
    assert tl.attn_timeline_layout(ctypes.byref(ev), ctypes.byref(mw)) == 0
    assert (ev.value, mw.value) == (8, 1 << 16)
    assert tl.attn_timeline_layout(None, ctypes.byref(mw)) == _lib.MGQA_ERR_NULL
    tl.attn_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    assert tl.attn_timeline_read(None, 1) == _lib.MGQA_ERR_NULL
    buf = (ctypes.c_ulonglong * 1)()
    assert tl.attn_timeline_read(buf, (1 << 16) * 9 + 1) == _lib.MGQA_ERR_RANGE


def test_version_and_error_strings():
    assert _lib.attn_version() == 104
    for code in range(-11, 1):
        s = _lib.error_string(code)
        assert s and s != "unknown error code"
    assert _lib.error_string(-99) == "unknown error code"


# Fake, 16-byte aligned, never dereferenced: every call below must fail
# validation before anything reaches the GPU.
P = ctypes.c_void_p(0x100000)
MIS = ctypes.c_void_p(0x100008)


def _ex(**kw):
    a = dict(q=P, k=P, v=P, out=P, B=1, Hq=4, Hkv=1, Lq=64, Lkv=64, d=128, causal=1, window=0,
             softcap=0.0, dtype=0, ws=None, wsb=0)
    a.update(kw)
    return _lib.attn_fwd_ex(a["q"], a["k"], a["v"], a["out"], a["B"], a["Hq"], a["Hkv"], a["Lq"],
                            a["Lkv"], a["d"], a["causal"], a["window"], a["softcap"], a["dtype"],
                            a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.MGQA_ERR_NULL),
    (dict(out=None), _lib.MGQA_ERR_NULL),
    (dict(B=0), _lib.MGQA_ERR_SHAPE),
    (dict(Lq=-1), _lib.MGQA_ERR_SHAPE),
    (dict(Hq=6, Hkv=4), _lib.MGQA_ERR_SHAPE),
    (dict(Hq=34, Hkv=2), _lib.MGQA_ERR_SHAPE),      # G = 17 > 16
    (dict(d=100), _lib.MGQA_ERR_HEAD_DIM),
    (dict(d=136), _lib.MGQA_ERR_HEAD_DIM),
    (dict(causal=2), _lib.MGQA_ERR_MASK),
    (dict(window=-1), _lib.MGQA_ERR_MASK),
    (dict(Lq=65, Lkv=64), _lib.MGQA_ERR_MASK),       # causal with Lq > Lkv
    (dict(Lq=65, Lkv=64, causal=0, window=8), _lib.MGQA_ERR_MASK),
    (dict(softcap=-1.0), _lib.MGQA_ERR_SOFTCAP),
    (dict(softcap=float("nan")), _lib.MGQA_ERR_SOFTCAP),
    (dict(softcap=float("inf")), _lib.MGQA_ERR_SOFTCAP),
    (dict(dtype=2), _lib.MGQA_ERR_DTYPE),
    (dict(q=MIS), _lib.MGQA_ERR_ALIGN),
    (dict(v=MIS), _lib.MGQA_ERR_ALIGN),
    # decode shape that needs a workspace, none given
    (dict(Hq=32, Hkv=8, Lq=1, Lkv=8192, B=8), _lib.MGQA_ERR_WORKSPACE),
    (dict(Hq=32, Hkv=8, Lq=1, Lkv=8192, B=8, ws=P, wsb=16), _lib.MGQA_ERR_WORKSPACE),
    (dict(Hq=32, Hkv=8, Lq=1, Lkv=8192, B=8, ws=ctypes.c_void_p(0x100010), wsb=1 << 30),
     _lib.MGQA_ERR_ALIGN),
])
def test_validation_codes(kw, code):
    assert _ex(**kw) == code


def test_cache_entry_point_validation_codes():
    f = _lib.attn_fwd_cache
    args = dict(B=1, Hq=16, Hkv=1, Lq=1, S=4096, length=4096, ring=-1, d=128, causal=1, W=0, cap=0.0,
                dt=0)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return f(P, P, P, P, a["B"], a["Hq"], a["Hkv"], a["Lq"], a["S"], a["length"], a["ring"],
                 a["d"], a["causal"], a["W"], a["cap"], a["dt"], None, 0, None)
    assert call(length=4097) == _lib.MGQA_ERR_RANGE        # length > S
    assert call(length=0) == _lib.MGQA_ERR_SHAPE
    assert call(ring=4096) == _lib.MGQA_ERR_RANGE          # ring start outside the cache
    assert call(ring=-2) == _lib.MGQA_ERR_RANGE
    assert call(Lq=64, Hq=4, ring=5) == _lib.MGQA_ERR_UNSUPPORTED  # ring needs the decode path
    assert call() == _lib.MGQA_ERR_WORKSPACE               # split decode without workspace
    assert f(None, P, P, P, 1, 16, 1, 1, 64, 64, -1, 128, 1, 0, 0.0, 0, None, 0, None) == _lib.MGQA_ERR_NULL


def test_cache_append_entry_point_validation_codes():
    f = _lib.attn_fwd_cache_append

    def call(q=P, kc=P, vc=P, nk=P, nv=P, out=P, B=1, Hq=8, Hkv=2, Lq=1, S=4096, pos=100, ring=-1,
             d=128, causal=1, W=0, cap=0.0, dt=0, ws=None, wsb=0):
        return f(q, kc, vc, nk, nv, out, B, Hq, Hkv, Lq, S, pos, ring, d, causal, W, cap, dt, ws, wsb,
                 None)
    assert call(nk=None) == _lib.MGQA_ERR_NULL
    assert call(nv=None) == _lib.MGQA_ERR_NULL
    assert call(S=0) == _lib.MGQA_ERR_SHAPE
    assert call(pos=-1) == _lib.MGQA_ERR_RANGE
    assert call(pos=4096) == _lib.MGQA_ERR_RANGE             # position + Lq > S
    assert call(Lq=4, pos=4093) == _lib.MGQA_ERR_RANGE
    assert call(S=(1 << 23) + 1) == _lib.MGQA_ERR_RANGE      # unit above 2^30 elements
    assert call(d=100) == _lib.MGQA_ERR_HEAD_DIM
    assert call(nk=MIS) == _lib.MGQA_ERR_ALIGN
    assert call(nv=MIS) == _lib.MGQA_ERR_ALIGN
    assert call(Hkv=8, Hq=32, B=8, pos=8191, S=8192) == _lib.MGQA_ERR_WORKSPACE  # split decode
    assert call(dt=2) == _lib.MGQA_ERR_DTYPE
    assert call(ring=4096) == _lib.MGQA_ERR_RANGE            # ring start outside the cache
    assert call(ring=-2) == _lib.MGQA_ERR_RANGE
    assert call(Lq=64, Hq=4, Hkv=4, ring=3, pos=1000) == _lib.MGQA_ERR_UNSUPPORTED  # ring needs decode


def test_append_validation_codes():
    g = _lib.kv_cache_append
    assert g(None, P, P, P, 1, 8, 1, 4, 2, 0, 2, 0, None, None) == _lib.MGQA_ERR_NULL
    assert g(P, P, P, P, 1, 8, 1, 4, 2, 7, 2, 0, None, None) == _lib.MGQA_ERR_RANGE   # pos > S-L
    assert g(P, P, P, P, 1, 8, 1, 4, 2, -1, 2, 0, None, None) == _lib.MGQA_ERR_RANGE
    assert g(P, P, P, P, 1, 8, 1, 4, 9, 0, 2, 0, None, None) == _lib.MGQA_ERR_RANGE   # L > S
    assert g(P, P, P, P, 1, 8, 1, 4, 2, 0, 3, 0, None, None) == _lib.MGQA_ERR_DTYPE
    assert g(P, P, P, P, 1, 8, 1, 4, 2, 0, 2, 2, None, None) == _lib.MGQA_ERR_SHAPE   # layout
    assert g(P, P, P, P, 0, 8, 1, 4, 2, 0, 2, 0, None, None) == _lib.MGQA_ERR_SHAPE


def test_attn_fwd_validation_codes():
    assert _lib.attn_fwd(None, P, P, P, 1, 4, 1, 64, 64, 128, 1, 0, 0.0, None) == _lib.MGQA_ERR_NULL
    assert _lib.attn_fwd(P, P, P, P, 1, 4, 1, 64, 64, 100, 1, 0, 0.0, None) == _lib.MGQA_ERR_HEAD_DIM
    assert _lib.attn_fwd(P, P, P, MIS, 1, 4, 1, 64, 64, 128, 1, 0, 0.0, None) == _lib.MGQA_ERR_ALIGN


def test_unit_size_limit():
    # One K/V unit (batch row, kv head) may hold at most 2^30 elements: the
    # kernels address it with 32-bit byte offsets and keep offset 2^31 for
    # "outside the range".
    for d in (128, 120, 64, 8):
        top = (1 << 30) // d
        assert _lib.attn_plan(1, 8, 1, 1, top, d, 1, 0, 0.0)[0] == 0
        assert _lib.attn_plan(1, 8, 1, 1, top + 1, d, 1, 0, 0.0)[0] == _lib.MGQA_ERR_RANGE
    assert _lib.attn_plan(2, 8, 2, 1, 1 << 23, 128, 0, 0, 0.0)[0] == 0   # many units at the limit
    f = _lib.attn_fwd_cache
    ws = ctypes.c_void_p(0x100000)
    for S, code in (((1 << 23) + 1, _lib.MGQA_ERR_RANGE), (1 << 23, _lib.MGQA_ERR_WORKSPACE)):
        assert f(P, P, P, P, 1, 16, 1, 1, S, 4096, -1, 128, 1, 0, 0.0, 0, None, 0, None) == code
    assert f(P, P, P, P, 1, 16, 1, 1, (1 << 23) + 1, 4096, -1, 128, 1, 0, 0.0, 0, ws, 1 << 30,
             None) == _lib.MGQA_ERR_RANGE


def test_non_causal_longer_query_is_allowed_in_plan():
    # No mask and no window: every key is visible to every row, Lq > Lkv is fine.
    rc, info = _lib.attn_plan(1, 2, 1, 100, 10, 64, 0, 0, 0.0)
    assert rc == 0 and info["workgroups"] >= 1


def test_plans_for_workloads():
    paths = {}
    for name, w in WORKLOADS.items():
        rc, info = _lib.attn_plan(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window,
                                  w.softcap, 1 if w.dtype == "fp16" else 0)
        assert rc == 0, name
        paths[name] = info
        assert info["workgroups"] >= 1
        assert info["d_qk_pad"] >= w.d and info["d_pv_pad"] >= w.d
        ws = _lib.attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window)
        assert ws == info["workspace_bytes"]
    assert paths["decode_gqa4_kv8192"]["path"] == 1
    assert paths["decode_gqa4_kv8192"]["nsplit"] > 1
    assert paths["decode_gqa16_kv32768_w4096_cap30"]["path"] == 1
    assert paths["prefill_gqa8_L4096_w1024_cap50"]["path"] == 0
    assert paths["encoder_siglip_L729_d72"]["path"] == 2
    assert paths["encoder_siglip_L729_d72"]["d_pv_pad"] == 80
    assert paths["encoder_siglip_L729_d72"]["d_qk_pad"] == 96
    # The decode band of the windowed decode covers only the last 4096 keys:
    # its splits times keys per split must not exceed the window plus a tile.
    info = paths["decode_gqa16_kv32768_w4096_cap30"]
    w = WORKLOADS["decode_gqa16_kv32768_w4096_cap30"]
    assert info["workgroups"] == w.B * w.Hkv * info["nsplit"] * info["ncol"]
    assert info["ncol"] == 2  # one 16-row block per unit with many key splits: column halves


def test_workspace_layout_fits():
    # The workspace covers the fixed 1 KiB counter block plus partials for
    # every position block, split, row and padded column.
    for (B, Hq, Hkv, Lq, Lkv, d, causal) in [(8, 32, 8, 1, 8192, 128, 1), (4, 64, 4, 1, 32768, 128, 1),
                                             (3, 12, 4, 4, 5000, 72, 1), (1, 16, 1, 1, 129, 64, 1),
                                             (2, 16, 2, 100, 333, 128, 1), (1, 8, 2, 16, 2000, 64, 1),
                                             (1, 3, 3, 150, 150, 72, 0)]:
        rc, info = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, d, causal, 0, 0.0)
        assert rc == 0
        if info["nsplit"] > 1:
            G = Hq // Hkv
            rows = info["rows_per_wg"]
            groups = info["workgroups"] // (info["nsplit"] * info["ncol"])
            assert groups * info["ncol"] <= 256  # the counters fit the fixed block
            m = min(rows // G, Lq)
            # O rows of the full padded width, (max, sum) per column slice
            need = 1024 + groups * info["nsplit"] * m * G * (info["d_pv_pad"] + 2 * info["ncol"]) * 4
            assert info["workspace_bytes"] >= need
        else:
            assert info["workspace_bytes"] == 0


def test_encoder_shapes_split_keys_when_row_blocks_are_few():
    """Short non-causal sequences with few heads: with a band of at most 768
    keys they run on the short-band kernel whatever the workgroup count (its
    eight waves split the band); with a longer band, row blocks alone would
    leave most compute units idle, so the plan splits the key axis across
    workgroups; with 16 heads the row blocks already fill the chip."""
    for H in (1, 2, 4, 8, 16):
        rc, info = _lib.attn_plan(1, H, H, 729, 729, 72, 0, 0, 0.0)
        assert rc == 0 and info["path"] == 2 and info["nsplit"] == 1, (H, info)
        assert info["workgroups"] == 16 * H and info["rows_per_wg"] == 48, (H, info)
    for H in (1, 2, 4):
        rc, info = _lib.attn_plan(1, H, H, 1000, 1000, 72, 0, 0, 0.0)
        assert rc == 0 and info["path"] == 1 and info["nsplit"] > 1, (H, info)
        assert info["workgroups"] >= 256 or info["nsplit"] > 1, (H, info)
    # A two-sided window short enough for the kernel keeps long sequences on it.
    rc, info = _lib.attn_plan(2, 2, 2, 1100, 1100, 72, 0, 300, 0.0)
    assert rc == 0 and info["path"] == 2, info


def test_column_halves_plan():
    """Many key splits of a single 16-row block: two workgroups per key range,
    each with half of the head size for P.V; never for other head sizes,
    several row blocks, or few splits."""
    rc, info = _lib.attn_plan(1, 8, 2, 4, 6000, 128, 1, 0, 20.0)   # 16 rows, long band
    assert rc == 0 and info["ncol"] == 2 and info["nsplit"] >= 4, info
    assert info["workgroups"] == 2 * info["nsplit"] * info["ncol"]
    rc, info = _lib.attn_plan(8, 32, 8, 1, 8192, 128, 1, 0, 0.0)   # 4 splits: no halves
    assert rc == 0 and info["ncol"] == 1, info
    rc, info = _lib.attn_plan(1, 16, 1, 1, 8192, 96, 1, 0, 0.0)    # head size 96: no halves
    assert rc == 0 and info["ncol"] == 1, info
    rc, info = _lib.attn_plan(1, 32, 2, 2, 8192, 128, 1, 0, 0.0)   # 32 rows a unit: no halves
    assert rc == 0 and info["ncol"] == 1, info
    rc, info = _lib.attn_plan(1, 2, 1, 300, 300, 128, 1, 0, 0.0)   # prefill-like: no halves
    assert rc == 0 and info["ncol"] == 1, info


def test_wide_split_plan():
    """A single 16-row block with at least eight 128-key tiles per workgroup
    runs 8 waves over 256-key tiles; few tiles per workgroup, two, three or
    four row blocks or column halves keep 4 waves over 128-key tiles (three
    row blocks over short bands take the short-band kernel)."""
    rc, info = _lib.attn_plan(8, 32, 8, 1, 8192, 128, 1, 0, 0.0)     # 4 splits of 16 tiles
    assert rc == 0 and info["keys_per_tile"] == 256 and info["ncol"] == 1, info
    rc, info = _lib.attn_plan(64, 64, 8, 1, 3000, 72, 1, 0, 0.0)     # no split, 24 tiles
    assert rc == 0 and info["keys_per_tile"] == 256 and info["nsplit"] == 1, info
    rc, info = _lib.attn_plan(4, 64, 4, 1, 32768, 128, 1, 4096, 30.0)  # column halves
    assert rc == 0 and info["keys_per_tile"] == 128 and info["ncol"] == 2, info
    rc, info = _lib.attn_plan(1, 4, 1, 64, 64, 128, 1, 0, 0.0)         # one tile
    assert rc == 0 and info["keys_per_tile"] == 128, info
    rc, info = _lib.attn_plan(1, 16, 16, 729, 1500, 72, 1, 0, 0.0)     # 48-row blocks, long band
    assert rc == 0 and info["path"] == 1 and info["keys_per_tile"] == 128 and info["rows_per_wg"] == 48, info
    rc, info = _lib.attn_plan(1, 16, 16, 700, 900, 80, 1, 0, 0.0)      # 32-row blocks, long band
    assert rc == 0 and info["keys_per_tile"] == 128 and info["rows_per_wg"] == 32, info
    rc, info = _lib.attn_plan(1, 48, 16, 729, 729, 40, 1, 0, 0.0)      # 64-row blocks
    assert rc == 0 and info["keys_per_tile"] == 128 and info["rows_per_wg"] == 64, info


def test_short_band_plan():
    """Three 16-row blocks over an unsplit band of at most 768 keys and head
    sizes 49..96 take the short-band kernel (path 2, no workspace, 96 keys per
    wave at most), also with few heads; longer bands and head size 48 or 128
    do not, and neither do decode rows that fit one split-KV workgroup."""
    def plan(*a):
        rc, info = _lib.attn_plan(*a)
        assert rc == 0, a
        return info
    for d in (56, 64, 72, 80, 88, 96):
        info = plan(1, 16, 16, 729, 729, d, 0, 0, 0.0)
        assert info["path"] == 2 and info["rows_per_wg"] == 48 and info["keys_per_tile"] == 96, (d, info)
        assert info["workspace_bytes"] == 0 and info["nsplit"] == 1 and info["workgroups"] == 256, (d, info)
        assert info["d_qk_pad"] == 32 * ((d + 31) // 32), (d, info)
    assert plan(1, 16, 16, 729, 729, 48, 0, 0, 0.0)["path"] == 1
    assert plan(1, 16, 16, 729, 729, 128, 0, 0, 0.0)["path"] == 1
    assert plan(1, 16, 16, 729, 768, 72, 1, 0, 0.0)["path"] == 2     # band of exactly 768 keys
    assert plan(1, 16, 16, 729, 769, 72, 1, 0, 0.0)["path"] == 1     # 769 keys: 25 steps
    assert plan(1, 4, 4, 729, 729, 72, 0, 0, 0.0)["path"] == 2       # few heads: waves split the band
    assert plan(8, 32, 8, 4, 700, 72, 1, 0, 0.0)["path"] == 1        # 16 rows per unit: split-KV
    assert plan(1, 16, 8, 800, 800, 80, 1, 300, 30.0)["path"] == 2   # two heads per kv head
    # ring buffers need the decode path
    P = ctypes.c_void_p(0x100000)
    rc = _lib.attn_fwd_cache(P, P, P, P, 1, 16, 16, 729, 729, 729, 5, 72, 0, 0, 0.0, 0, None, 0, None)
    assert rc == _lib.MGQA_ERR_UNSUPPORTED


def test_noalloc_scratch_covers_every_plan():
    """attn_fwd_noalloc serves split plans from a fixed device array: every
    plan over a sweep of decode, multi-token and short shapes fits it, and
    validation errors come before any HIP call."""
    worst = 0
    for B in (1, 8, 64):
        for Hkv in (1, 2, 8):
            for G in (1, 4, 16):
                for Lq in (1, 4, 16, 48):
                    for d in (64, 96, 128):
                        for Lkv in (4096, 1 << 20):
                            rc, info = _lib.attn_plan(B, G * Hkv, Hkv, Lq, Lkv, d, 1, 0, 0.0)
                            if rc == 0:
                                worst = max(worst, info["workspace_bytes"])
    assert 0 < worst <= _lib.MGQA_NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p(0x100000)
    assert _lib.attn_fwd_noalloc(None, P, P, P, 1, 4, 1, 1, 64, 128, 1, 0, 0.0, 0, None) == _lib.MGQA_ERR_NULL
    assert _lib.attn_fwd_noalloc(P, P, P, P, 1, 4, 3, 1, 64, 128, 1, 0, 0.0, 0, None) == _lib.MGQA_ERR_SHAPE
    assert _lib.attn_fwd_noalloc(P, P, P, ctypes.c_void_p(0x100008), 1, 4, 1, 1, 64, 128, 1, 0, 0.0, 0,
                                 None) == _lib.MGQA_ERR_ALIGN


def _pipe_item_positions(info, B, Hq, Hkv, Lq):
    """Query positions each work item of one unit covers, decoded from the
    plan's item layout the way the head-size-128 prefill kernel decodes it."""
    G = Hq // Hkv
    m = info["rows_per_wg"] // G
    n = -(-Lq // m)
    items = info["workgroups"] // (B * Hkv)
    assert items * B * Hkv == info["workgroups"]
    pairs, ramp, full = info["pf_pairs"], info["pf_ramp"], info["pf_full"]
    assert pairs == (ramp + 1) // 2 and full >= 0
    halves = items - pairs - full
    assert halves >= 0 and halves % 2 == 0
    if halves:
        assert m % 2 == 0
    out = []
    for j in range(items):
        if j < pairs:
            blocks = [ramp - 1 - j] + ([j] if j < ramp - 1 - j else [])
            out.append([p for pb in blocks for p in range(pb * m, min(Lq, pb * m + m))])
        elif j < pairs + full:
            pb = n - 1 - (j - pairs)
            out.append(list(range(pb * m, min(Lq, pb * m + m))))
        else:
            h = j - pairs - full
            pb = n - 1 - full - (h >> 1)
            q0 = pb * m + (h & 1) * (m // 2)
            out.append(list(range(q0, min(Lq, q0 + m // 2))))
    return out


@pytest.mark.parametrize("shape", [
    (2, 32, 4, 4096, 4096, 1, 1024),   # windowed causal: ramp halved
    (2, 32, 4, 4096, 4096, 1, 0),      # causal
    (2, 32, 4, 4096, 4096, 0, 0),      # no mask
    (1, 64, 4, 4096, 4096, 1, 0),      # fewer units than XCDs: ramp paired
    (1, 8, 1, 32768, 32768, 1, 0),     # one unit
    (1, 16, 16, 4096, 4096, 1, 0),     # 128 positions per block
    (2, 32, 4, 1000, 1000, 1, 0),      # partial last block
    (2, 24, 8, 3001, 3001, 1, 700),    # G = 3: odd blocks of 42 positions
    (2, 32, 4, 2048, 4096, 1, 1024),   # queries at the end of a longer key range
    (4, 32, 8, 2048, 2048, 1, 512),
    (3, 40, 5, 2500, 2500, 0, 300),    # bidirectional window
])
def test_prefill_items_cover_every_position_once(shape):
    """The head-size-128 prefill plan splits each (batch row, kv head) into
    work items -- ramp pairs, whole blocks, half blocks -- that together hold
    every query position exactly once and no empty item."""
    B, Hq, Hkv, Lq, Lkv, causal, window = shape
    rc, info = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, 128, causal, window, 0.0)
    assert rc == 0 and info["path"] == 0, info
    items = _pipe_item_positions(info, B, Hq, Hkv, Lq)
    assert all(items), "empty work item"
    flat = sorted(p for it in items for p in it)
    assert flat == list(range(Lq)), shape
    # The same shape with another head size takes the generic prefill kernel
    # with one whole block per workgroup and no item layout.
    rc, other = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, 96, causal, window, 0.0)
    assert rc == 0 and (other["pf_pairs"], other["pf_ramp"], other["pf_full"]) == (0, 0, 0)


def test_prefill_item_layouts_chosen():
    """Which layout the launch model picks for four prefill shapes: a causal
    prefill with fewer units (batch rows x kv heads) than XCDs pairs the
    ramp's ends, so every XCD gets an even share; a causal prefill of 128-
    position blocks that fills one round halves every block; the windowed
    causal prefill of 2 x 4 kv heads and an unmasked prefill keep one block
    per workgroup, last first."""
    rc, info = _lib.attn_plan(1, 64, 4, 4096, 4096, 128, 1, 0, 0.0)
    assert info["pf_pairs"] > 0 and info["pf_ramp"] >= 2 * info["pf_pairs"] - 1
    rc, info = _lib.attn_plan(1, 16, 16, 4096, 4096, 128, 1, 0, 0.0)
    assert (info["pf_pairs"], info["pf_full"], info["workgroups"]) == (0, 0, 16 * 64)
    for causal, window in ((1, 1024), (0, 0)):
        rc, info = _lib.attn_plan(2, 32, 4, 4096, 4096, 128, causal, window, 50.0)
        assert (info["pf_pairs"], info["pf_ramp"], info["pf_full"], info["workgroups"]) == (0, 0, 256, 8 * 256)


def test_gpu_sweep_reaches_every_plan_form():
    """The seeded GPU sweep's shapes (fixed by its generator seeds) reach every
    form the planner can pick, so the sweep checks each against the oracle."""
    from .test_gpu_sweep import SHAPES
    forms = set()
    for i, B, Hq, Hkv, Lq, Lkv, d, causal, window, cap, dt in SHAPES:
        rc, p = _lib.attn_plan(B, Hq, Hkv, Lq, Lkv, d, int(causal), window, cap, 0 if dt == "bf16" else 1)
        assert rc == 0
        if p["path"] == 0 and d == 128:
            items = p["workgroups"] // (B * Hkv)
            forms.add("pipe_pairs" if p["pf_pairs"] else "pipe")
            if items > p["pf_pairs"] + p["pf_full"]:
                forms.add("pipe_halves")
        elif p["path"] == 0:
            forms.add(f"prefill_rows_{p['rows_per_wg']}")
        elif p["path"] == 2:
            forms.add("short_band")
        else:
            forms.add("split")
            if p["nsplit"] > 1:
                forms.add("key_splits")
            if p["keys_per_tile"] == 256:
                forms.add("wide")
            if p["ncol"] == 2:
                forms.add("column_halves")
            forms.add(f"split_rows_{p['rows_per_wg']}")
    want = {"pipe", "pipe_pairs", "pipe_halves", "prefill_rows_256", "prefill_rows_128", "short_band", "split", "key_splits", "wide",
            "column_halves", "split_rows_16", "split_rows_32", "split_rows_48"}
    assert want <= forms, want - forms
