"""bench.py on a machine without a GPU: a run on more than one GPU is refused
with a message (the library has no multi-GPU path), before any GPU work; and
the units of the prefill's secondary (transcendental) roofline."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_names_the_timing_contract():
    r = _run("--help")
    assert r.returncode == 0
    assert "exactly K calls" in r.stdout


def test_transcendental_roofline_units():
    """The secondary roofline of the softcapped prefill: three transcendental
    instructions per in-band pair with a softcap (exp and reciprocal for tanh,
    exp for the softmax), one without; peak = 256 CUs x 4 SIMDs x 8 lanes per
    clock x 2.4 GHz."""
    import bench
    from masked_gqa_attention_amd import accounting, synth
    assert bench.trans_ops_per_pair(50.0) == 3 and bench.trans_ops_per_pair(0.0) == 1
    assert abs(bench.TRANS_PEAK_TOPS - 19.6608) < 1e-9
    w = synth.WORKLOADS["prefill_gqa8_L4096_w1024_cap50"]
    pairs = accounting.workload_work(w)["flops"] / (4 * w.d)
    assert pairs == 234_913_792  # B*Hq * (W(W+1)/2 + (L-W)W) with W = 1024, L = 4096
    # at the peak, the transcendentals alone take ~35.8 us per launch
    assert 35.8 < 3 * pairs / (bench.TRANS_PEAK_TOPS * 1e12) * 1e6 < 35.9
