#!/usr/bin/env python3
"""Benchmark of the masked GQA attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workloads a,b] [--no-cpu-baseline] [--no-cache-step]

A step is one attention call (one pass of the whole path: band plan, K/V
staging, Q.K^T, softcap, mask, online softmax, P.V, epilogue, and for decode
the split partials and their fixed-order merge) over one batch of seeded
synthetic input already resident in HBM.  The headline workload is the GQA
4:1 decode over 8192 cached keys (B=8, Hq=32, Hkv=8, d=128), reported in
GB/s of algorithmic bytes; the other workloads are measured the same way and
listed under "workloads" (TFLOP/s for prefill/encoder, GB/s for decode).
Three extension shapes are measured the same way under "next_rows": a
multi-token decode, an encoder with few heads (key splits) and the long
windowed decode over a ring-buffer cache.
The two decode workloads are also timed as a step over a KV cache
("cache_step": the new rows written by kv_cache_append and then attended by
attn_fwd_cache, against the one fused attn_fwd_cache_append call).

Timing: W untimed calls, then exactly K calls between two HIP events on the
stream the kernels run on, bracketed by device synchronisation; that rate is
the reported value.  Each workload's record also holds its error against the
float64 oracle on every output element (max abs/rel error, allclose at
rtol = atol = 2e-2), whether three calls on the same input gave the same
bytes, and the oracle's own time on this host's cores (a process pool with
one worker per core of the affinity mask, started before the GPU is used).  Each workload is then also timed in 30 rounds of at
least 1 ms of back-to-back calls ("spread": median, 10th and 90th percentile
of the per-call time over the rounds).  Inputs
rotate over several copies so that repeated calls stream from HBM rather than
from the 256 MB last-level cache.  Prints ONE JSON line.
Besides "roofline" (the headline decode against HBM) the line carries
"roofline_prefill" (the windowed softcapped prefill against the bf16 MFMA
peak) and "roofline_prefill_trans" (the same launches against the
transcendental unit: three transcendental instructions per in-band pair with
the softcap, one without, over a peak of a quarter of the fp32 lane rate).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import re
import os
import shutil
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HEADLINE = "decode_gqa4_kv8192"
METRIC = "attention TFLOP/s (prefill) + KV GB/s (decode), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 / fp16 MFMA
# Transcendental instructions (v_exp_f32, v_rcp_f32): a quarter of the fp32
# vector lane rate, i.e. 8 lanes per clock per SIMD: 256 CUs x 4 SIMDs x 8 x
# 2.4 GHz, in tera-operations per second.
TRANS_PEAK_TOPS = 256 * 4 * 8 * 2.4e9 / 1e12


def trans_ops_per_pair(softcap: float) -> int:
    """Transcendental instructions the method needs per in-band (query, key)
    pair on this chip, which has no tanh instruction: the softmax exponential,
    plus for the softcap c*tanh(s/c) = c - 2c/(exp(2s/c) + 1) one exponential
    and one reciprocal."""
    return 3 if softcap > 0 else 1
LLC_BYTES = 256 * 1024 * 1024    # MI355X last-level (Infinity) cache
COPY_BYTES = 256 * 1024 * 1024   # plain copy used to calibrate byte counters
KERNEL_SRC = os.path.join(ROOT, "masked_gqa_attention_amd", "csrc", "mgqa_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_splitkv_kernel_decode_gqa4_kv8192.json")
TRAFFIC_FILE_PREFILL = os.path.join(ROOT, "profiles",
                                    "traffic_prefill_pipe4_kernel_prefill_gqa8_L4096_w1024_cap50.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


class Runner:
    """Device copies of one workload and a lean C-ABI call per copy."""

    def __init__(self, w, copies):
        import torch
        from masked_gqa_attention_amd import _lib, synth
        self.torch = torch
        self.w = w
        q, k, v = synth.draw_qkv(w)
        self.host = (q, k, v)
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        np_int = "int16"

        def dev(a):
            if w.dtype == "bf16":
                return torch.from_numpy(a.view(np_int)).view(torch.bfloat16).cuda()
            return torch.from_numpy(a).cuda()

        base = [dev(a) for a in (q, k, v)]
        self.sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
        self.outs = [torch.empty_like(base[0]) for _ in range(copies)]
        self.ws_bytes = _lib.attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d,
                                                  int(w.causal), w.window)
        self.ws = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream().cuda_stream
        self.fn = _lib.load().attn_fwd_ex
        dtype_code = _lib.MGQA_BF16 if w.dtype == "bf16" else _lib.MGQA_FP16
        self.args = []
        for (tq, tk, tv), to in zip(self.sets, self.outs):
            self.args.append((tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(),
                              w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window,
                              ctypes.c_float(w.softcap), dtype_code,
                              self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes,
                              self.stream))
        del dt

    def call(self, i):
        rc = self.fn(*self.args[i % len(self.args)])
        if rc != 0:
            from masked_gqa_attention_amd import _lib
            raise RuntimeError(f"attn_fwd_ex failed: {_lib.error_string(rc)}")

    def time(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.call(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            self.call(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps  # ms per call

    def spread(self, ms_est, rounds=30, min_round_ms=1.0):
        """Per-call time over `rounds` rounds of back-to-back calls, each round
        at least `min_round_ms` long and timed by its own pair of HIP events
        on the launch stream: median, 10th and 90th percentile."""
        torch = self.torch
        n = max(1, int(-(-min_round_ms // max(ms_est, 1e-6))))
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(rounds)]
        torch.cuda.synchronize()
        i = 0
        for a, b in ev:
            a.record()
            for _ in range(n):
                self.call(i)
                i += 1
            b.record()
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) / n for a, b in ev)
        pct = lambda f: per[min(rounds - 1, int(round(f * (rounds - 1))))]
        return {"rounds": rounds, "calls_per_round": n,
                "p10_ms": pct(0.1), "median_ms": pct(0.5), "p90_ms": pct(0.9)}

    def output_f64(self, i=0):
        from masked_gqa_attention_amd import synth
        o = self.outs[i % len(self.outs)]
        torch = self.torch
        if self.w.dtype == "bf16":
            arr = o.view(torch.int16).cpu().numpy().view("uint16")
        else:
            arr = o.cpu().numpy()
        return synth.storage_to_f64(arr, self.w.dtype)


class RingRunner(Runner):
    """A decode over a ring-buffer KV cache of Lkv slots holding Lkv logical
    keys (logical key j in slot (RING_START + j) mod Lkv), through
    attn_fwd_cache; the copies rotate like Runner's."""

    def __init__(self, w, copies):
        super().__init__(w, copies)
        from masked_gqa_attention_amd import _lib, synth
        self.fn = _lib.load().attn_fwd_cache
        dtype_code = _lib.MGQA_BF16 if w.dtype == "bf16" else _lib.MGQA_FP16
        self.args = [(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(),
                      w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.Lkv, synth.RING_START, w.d, int(w.causal),
                      w.window, ctypes.c_float(w.softcap), dtype_code,
                      self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, self.stream)
                     for (tq, tk, tv), to in zip(self.sets, self.outs)]

    def call(self, i):
        rc = self.fn(*self.args[i % len(self.args)])
        if rc != 0:
            from masked_gqa_attention_amd import _lib
            raise RuntimeError(f"attn_fwd_cache failed: {_lib.error_string(rc)}")


# Decode workloads also timed as a step over a KV cache (new rows written, then attended).
CACHE_STEP_WORKLOADS = ("decode_gqa4_kv8192", "decode_gqa16_kv32768_w4096_cap30")


def cache_step(r, steps, warmup):
    """A decode step over a KV cache holding the workload's K/V (Lkv slots per
    batch row and kv head): the Lq new float32 key/value rows are written at
    position Lkv - Lq and the queries attend over all Lkv keys.  Timed as two
    calls (kv_cache_append, then attn_fwd_cache) and as the single fused call
    (attn_fwd_cache_append), on the runner's device copies (the caches), so
    the same bytes stream from HBM as in the attention-only timing."""
    import numpy as np
    from masked_gqa_attention_amd import _lib
    torch, w = r.torch, r.w
    lib = _lib.load()
    rng = np.random.default_rng(w.seed + 7)
    nk, nv = (torch.from_numpy(rng.standard_normal((w.B, w.Hkv, w.Lq, w.d), dtype=np.float32)).cuda()
              for _ in range(2))
    pos = w.Lkv - w.Lq
    dt = _lib.MGQA_BF16 if w.dtype == "bf16" else _lib.MGQA_FP16
    ws = r.ws.data_ptr() if r.ws_bytes else None
    cap = ctypes.c_float(w.softcap)
    outs = [torch.empty_like(t[0]) for t in r.sets]
    two, fused = [], []
    for (tq, tk, tv), to in zip(r.sets, outs):
        q, kc, vc, o = tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr()
        two.append(((kc, vc, nk.data_ptr(), nv.data_ptr(), w.B, w.Lkv, w.Hkv, w.d, w.Lq, pos, dt, 1, None,
                     r.stream),
                    (q, kc, vc, o, w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.Lkv, -1, w.d, int(w.causal), w.window,
                     cap, dt, ws, r.ws_bytes, r.stream)))
        fused.append((q, kc, vc, nk.data_ptr(), nv.data_ptr(), o, w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, pos, -1, w.d,
                      int(w.causal), w.window, cap, dt, ws, r.ws_bytes, r.stream))

    def call_two(i):
        a, b = two[i % len(two)]
        if lib.kv_cache_append(*a) != 0 or lib.attn_fwd_cache(*b) != 0:
            raise RuntimeError("cache update or attention failed")

    def call_fused(i):
        if lib.attn_fwd_cache_append(*fused[i % len(fused)]) != 0:
            raise RuntimeError("attn_fwd_cache_append failed")

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(steps):
            fn(i)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    t_two, t_fused = timed(call_two), timed(call_fused)
    fig = figures(w, t_fused)
    return {"new_rows": w.Lq, "position": pos, "cache_slots": w.Lkv, "steps": steps,
            "update_then_attention_ms": t_two, "fused_ms": t_fused,
            "fused_value": fig["value"], "unit": fig["unit"], "fused_frac": fig["frac"]}


def copies_for(w) -> int:
    """Input copies rotated through so that they total at least twice the
    last-level cache (never fewer than three)."""
    from masked_gqa_attention_amd import accounting
    touched = accounting.workload_work(w)["bytes"]
    return max(3, min(32, -(-2 * LLC_BYTES // max(touched, 1))))


def figures(w, ms):
    from masked_gqa_attention_amd import accounting
    wk = accounting.workload_work(w)
    decode = w.Lq * w.G <= 16
    if decode:
        gbs = wk["bytes"] / (ms * 1e-3) / 1e9
        return {"unit": "GB/s", "value": gbs, "bound": "hbm", "peak": HBM_PEAK_GBS,
                "frac": gbs / HBM_PEAK_GBS, "alg_bytes": wk["bytes"], "alg_flops": wk["flops"]}
    tf = wk["flops"] / (ms * 1e-3) / 1e12
    return {"unit": "TFLOP/s", "value": tf, "bound": "mfma", "peak": MFMA_PEAK_TFLOPS,
            "frac": tf / MFMA_PEAK_TFLOPS, "alg_bytes": wk["bytes"], "alg_flops": wk["flops"]}


def kernel_name(plan, w) -> str:
    """The attention kernel a plan launches (as in the library's dispatch)."""
    if plan.get("path") == 1:
        return "splitkv_kernel"
    if plan.get("path") == 2:
        return "encoder_kernel"
    return "prefill_pipe4_kernel" if w.d == 128 else "prefill_kernel"


def blas_config() -> str:
    """One line naming numpy's BLAS (the oracle's matrix products)."""
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{cfg.get('name')} {cfg.get('version')}"
    except Exception:  # pragma: no cover
        return "unknown"


def determinism(r) -> bool:
    """Three calls on the first input copy give the same output bytes."""
    torch = r.torch
    outs = []
    for _ in range(3):
        r.call(0)
        torch.cuda.synchronize()
        outs.append(r.outs[0].view(torch.int16).clone())
    return all(torch.equal(outs[0], o) for o in outs[1:])


def oracle_leg(pool, w, host, gpu_out, runs):
    """The float64 oracle, as it stands, on the workload's whole input, run
    head by head in the process pool: its wall time (median of `runs`) in the
    workload's algorithmic unit, and the GPU output's error against it on
    every element."""
    from masked_gqa_attention_amd import accounting, synth
    qf, kf, vf = (synth.storage_to_f64(a, w.dtype) for a in host)
    times, ref = [], None
    for _ in range(runs):
        ref, t = pool.timed_attention(qf, kf, vf, w.causal, w.window, w.softcap)
        times.append(t)
    t = sorted(times)[len(times) // 2]
    wk = accounting.workload_work(w)
    decode = w.Lq * w.G <= 16
    err = np.abs(gpu_out - ref)
    finite = bool(np.isfinite(gpu_out).all())
    return {
        "oracle": {"value": (wk["bytes"] / t / 1e9) if decode else (wk["flops"] / t / 1e9),
                   "unit": "GB/s" if decode else "GFLOP/s", "seconds": t, "runs": runs,
                   "cores": pool.workers, "kind": "oracle"},
        "parity": {"elements": int(gpu_out.size), "max_abs_err": float(err.max()),
                   "max_rel_err": float((err / np.maximum(np.abs(ref), 1e-6)).max()),
                   "nrmse": float(np.sqrt(np.mean(err ** 2)) / (np.sqrt(np.mean(ref ** 2)) or 1.0)),
                   "allclose": finite and bool((err <= 2e-2 + 2e-2 * np.abs(ref)).all()),
                   "rtol": 2e-2, "atol": 2e-2},
    }


def dispatch_floor_us(torch, n=2000) -> float:
    """Per-call time of back-to-back one-element fills on the current stream:
    the launch-to-launch floor any kernel of this library pays."""
    x = torch.zeros(1, device="cuda")
    for _ in range(50):
        x.fill_(1.0)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        x.fill_(1.0)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3


def device_info(torch) -> dict:
    props = torch.cuda.get_device_properties(0)
    info = {"name": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "max_sclk_mhz": (props.clock_rate / 1000.0) if getattr(props, "clock_rate", 0) else None,
            "sclk_now_mhz": None}
    # Shader clocks from rocm-smi in a child process (no GPU work of ours): the
    # current one (the card is idle by then) and the highest supported level.
    # --showclocks names its entries ("sclk clock speed:": "(2404Mhz)");
    # --showclkfrq lists the shader clock levels by number ("2": "2400Mhz").
    def smi_cmd():
        # rocm-smi is a Python script: run it with this interpreter, so that
        # no process replaces itself through its "env python3" line.
        path = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
        real = os.path.realpath(path)
        try:
            with open(real, "rb") as f:
                is_python = b"python" in f.readline()
        except OSError:
            is_python = False
        return [sys.executable, real] if is_python else [path]

    def smi_mhz(flag, want):
        r = subprocess.run(smi_cmd() + [flag, "--json"], capture_output=True, text=True, timeout=20)
        out = r.stdout[r.stdout.index("{"):] if "{" in r.stdout else "{}"
        found = []
        for card in json.loads(out).values():
            for key, val in card.items():
                m = re.search(r"(\d+(?:\.\d+)?)\s*mhz", str(val), re.I)
                if m and want(key):
                    found.append(float(m.group(1)))
        return found
    try:
        now = smi_mhz("--showclocks", lambda key: "sclk" in key.lower())
        info["sclk_now_mhz"] = now[0] if now else None
        levels = smi_mhz("--showclkfrq", lambda key: key.strip().isdigit())
        if levels:
            info["max_sclk_mhz"] = max(levels)
    except Exception:
        pass
    return info


def load_traffic(path=TRAFFIC_FILE):
    """Counter-derived HBM bytes per launch of a kernel (read + written, each
    counter scaled by a known-size copy), if the counters were taken on the
    current kernel source; otherwise None."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
    except Exception:
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="all",
                    help="comma list of extra workloads to measure besides the headline, or 'all'/'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle legs (oracle timing and the per-workload error against it)")
    ap.add_argument("--no-cache-step", action="store_true",
                    help="skip the decode-step-over-a-cache timings (update + attention, fused)")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the extension shapes (multi-token decode, few-head split-K encoder, "
                         "ring-buffer decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy 5 times (a known-size "
                         "reference for hardware byte counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (each "
              "(batch, kv head) unit is independent and could run on a GPU of its own). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    # The oracle's worker processes start before anything touches the GPU.
    pool = None
    if not args.no_cpu_baseline:
        from oracle.pool import OraclePool
        pool = OraclePool()
        log(f"oracle pool: {pool.workers} worker processes (host cores in the affinity mask)")

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from masked_gqa_attention_amd import _lib, synth
    _lib.load()

    names = [HEADLINE]
    if args.workloads == "all":
        names += [n for n in synth.WORKLOAD_ORDER if n != HEADLINE]
    elif args.workloads != "none":
        names += [n for n in args.workloads.split(",") if n and n != HEADLINE]

    floor = dispatch_floor_us(torch)
    log(f"dispatch floor (back-to-back one-element fills): {floor:.2f} us/call")

    results, kept = {}, {}
    headline = None
    for name in names:
        w = synth.WORKLOADS[name]
        copies = copies_for(w)
        log(f"{name}: {copies} input copies")
        r = Runner(w, copies)
        if name == HEADLINE:
            steps, warmup = args.steps, args.warmup
        else:
            r.call(0)
            torch.cuda.synchronize()
            est = r.time(3, 1)
            steps = int(max(10, min(2000, 200.0 / max(est, 1e-3))))
            warmup = max(3, steps // 10)
        ms = r.time(steps, warmup)
        fig = figures(w, ms)
        rc, plan = _lib.attn_plan(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window,
                                  w.softcap, 0 if w.dtype == "bf16" else 1)
        sp = r.spread(ms)
        same = determinism(r)
        results[name] = {"ms": ms, "steps": steps, "copies": copies, **fig,
                         "kernel": kernel_name(plan, w), "spread": sp, "memcmp_deterministic": same,
                         "plan": plan, "shape": w.describe()}
        log(f"{name}: {ms * 1e3:.2f} us/call  {fig['value']:.1f} {fig['unit']}  "
            f"({100 * fig['frac']:.1f}% of {fig['bound']} peak); rounds: median "
            f"{sp['median_ms'] * 1e3:.2f} us, p10 {sp['p10_ms'] * 1e3:.2f}, p90 {sp['p90_ms'] * 1e3:.2f}; "
            f"same bytes over 3 calls: {same}")
        if name in CACHE_STEP_WORKLOADS and not args.no_cache_step:
            st = cache_step(r, steps, warmup)
            results[name]["cache_step"] = st
            log(f"{name} as a cache step: update + attention {st['update_then_attention_ms'] * 1e3:.2f} us, "
                f"fused {st['fused_ms'] * 1e3:.2f} us")
        kept[name] = (w, r.host, r.output_f64(0))
        if name == HEADLINE:
            headline = (r, ms, steps, fig)
        else:
            del r
            torch.cuda.empty_cache()

    if not args.no_next_rows and args.workloads == "all":
        line_next = {}
        for name, w in synth.NEXT_WORKLOADS.items():
            copies = copies_for(w)
            r = (RingRunner if name.startswith("ring_") else Runner)(w, copies)
            r.call(0)
            torch.cuda.synchronize()
            est = r.time(3, 1)
            steps = int(max(10, min(2000, 200.0 / max(est, 1e-3))))
            ms = r.time(steps, max(3, steps // 10))
            fig = figures(w, ms)
            sp = r.spread(ms)
            rc, plan = _lib.attn_plan(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window,
                                      w.softcap, 0 if w.dtype == "bf16" else 1)
            line_next[name] = {"ms": ms, "steps": steps, "copies": copies, **fig,
                               "kernel": kernel_name(plan, w), "spread": sp, "plan": plan}
            log(f"{name}: {ms * 1e3:.2f} us/call  {fig['value']:.1f} {fig['unit']}  "
                f"({100 * fig['frac']:.1f}% of {fig['bound']} peak)")
            del r
            torch.cuda.empty_cache()
        results_next = line_next
    else:
        results_next = None

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 x {COPY_BYTES} bytes read + written")
        del src, dst

    dev = device_info(torch)
    r, ms, steps, fig = headline
    w = r.w
    traffic = load_traffic()
    line = {
        "metric": METRIC,
        "value": fig["value"],
        "unit": fig["unit"],
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V (PCG64, Q then K then V), resident in HBM",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq,
                   "Lkv": w.Lkv, "d": w.d, "causal": w.causal, "window": w.window,
                   "softcap": w.softcap, "seed": w.seed, "input_copies": len(r.outs)},
        "roofline": {"bound": "hbm", "achieved": fig["value"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": fig["frac"], "traffic": traffic,
                     "kernel": results[HEADLINE]["kernel"],
                     "alg_bytes_per_launch": fig["alg_bytes"]},
    }
    pre = "prefill_gqa8_L4096_w1024_cap50"
    if pre in results:
        rp = results[pre]
        line["roofline_prefill"] = {"bound": "mfma", "achieved": rp["value"], "peak": MFMA_PEAK_TFLOPS,
                                    "unit": "TFLOP/s", "frac": rp["frac"],
                                    "traffic": load_traffic(TRAFFIC_FILE_PREFILL),
                                    "kernel": rp["kernel"], "alg_flops_per_launch": rp["alg_flops"],
                                    "ms_per_launch": rp["ms"]}
        # Secondary roofline of the same launches: the transcendental unit.
        wp = synth.WORKLOADS[pre]
        ops = rp["alg_flops"] / (4 * wp.d) * trans_ops_per_pair(wp.softcap)
        tops = ops / (rp["ms"] * 1e-3) / 1e12
        line["roofline_prefill_trans"] = {"bound": "alu", "achieved": tops, "peak": TRANS_PEAK_TOPS,
                                          "unit": "Tops/s", "frac": tops / TRANS_PEAK_TOPS, "traffic": None,
                                          "kernel": rp["kernel"], "alg_ops_per_launch": ops,
                                          "ops_per_pair": trans_ops_per_pair(wp.softcap)}
    if pool is not None:
        log("oracle legs (every workload, whole input, process pool) ...")
        for name, (wk, host, gpu_out) in kept.items():
            leg = oracle_leg(pool, wk, host, gpu_out, runs=1 if wk.Lq * wk.Lkv >= (1 << 24) else 3)
            results[name].update(leg)
            log(f"{name}: oracle {leg['oracle']['seconds']:.3f} s on {pool.workers} processes; "
                f"max abs err {leg['parity']['max_abs_err']:.3e}, allclose {leg['parity']['allclose']}")
        pool.close()
        o = results[HEADLINE]["oracle"]
        line["cpu_baseline"] = {
            "value": o["value"], "unit": o["unit"], "cores": o["cores"], "kind": "oracle",
            "sample": f"whole {w.name} input ({w.B * w.Hq * w.Lq} query rows x {w.Lkv} keys), float64 oracle "
                      f"head by head in a pool of {o['cores']} processes, median of {o['runs']} runs",
            "seconds": o["seconds"], "blas": blas_config(),
        }
    else:
        line["cpu_baseline"] = None
    line.update({
        "workloads": {n: {k: v for k, v in res.items() if k not in ("shape",)} for n, res in results.items()},
        "next_rows": results_next,
        "dispatch_floor_us": floor,
        "device": dev,
        "host_cores": len(os.sched_getaffinity(0)),
        "torch": torch.__version__,
        "hip": torch.version.hip,
        "kernel_source_sha256": kernel_source_hash(),
    })
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
