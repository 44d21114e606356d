"""The timestamped measurement build (libmgqa_timeline.so) on every kernel:
each workload runs through `python -m masked_gqa_attention_amd.timeline` in a
child process (one process opens one build), which checks that every wave of
every recorded launch left a record with non-decreasing event times; the
output it saves must equal the library's own output bit for bit (the marks
move no arithmetic)."""
import os
import subprocess
import sys

import numpy as np
import pytest

from masked_gqa_attention_amd import _lib, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="no GPU")]

from .gpu_util import announce, to_device, to_host  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# workload, kernel form reached
CASES = [
    ("decode_gqa4_kv8192", "split-KV, 8 waves, 4 key splits"),
    ("decode_gqa16_kv32768_w4096_cap30", "split-KV, column halves, 8 key splits"),
    ("encoder_siglip_L729_d72", "short-band"),
    ("tiny_causal_gqa4_L64", "split-KV, one split"),
    ("prefill_gqa8_L4096_w1024_cap50", "pipelined head-size-128 prefill"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_timeline_build_records_and_bits(case, tmp_path):
    name, form = case
    if not os.path.exists(_lib.TIMELINE_LIB_PATH):
        pytest.fail(f"{_lib.TIMELINE_LIB_PATH} not built")
    announce(f"timeline {name} ({form})")
    saved = tmp_path / "out.npy"
    r = subprocess.run([sys.executable, "-m", "masked_gqa_attention_amd.timeline", name, "--launches", "2",
                        "--warmup", "1", "--check", "--save-output", str(saved)],
                       cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, f"{name}: exit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
    w = synth.WORKLOADS[name]
    q, k, v = synth.draw_qkv(w)
    tq, tk, tv = (to_device(a, w.dtype) for a in (q, k, v))
    from masked_gqa_attention_amd import api
    out = api.attn(tq, tk, tv, causal=w.causal, window=w.window, softcap=w.softcap)
    torch.cuda.synchronize()
    mine = to_host(out, w.dtype)
    theirs = np.load(saved)
    assert theirs.shape == mine.shape and theirs.dtype == mine.dtype
    diff = int((theirs != mine).sum())
    assert diff == 0, f"{name}: {diff} elements differ between the timeline build and the library"
