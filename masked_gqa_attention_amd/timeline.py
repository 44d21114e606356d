"""Where the time of one attention launch goes, per wave and per XCD.

    python -m masked_gqa_attention_amd.timeline WORKLOAD [--launches 5] [--warmup 3]
        [--check] [--save-output PATH] [--markdown PATH]

Runs a workload of synth.WORKLOADS / synth.NEXT_WORKLOADS (seeded synthetic
inputs, rotated over enough copies that they do not fit the last-level cache
together, as the benchmark does) through libmgqa_timeline.so, the
measurement build whose kernels timestamp named events per wave
(include/mgqa_timeline.h).  For each recorded launch it reports, in µs from
the first wave's start: per event the earliest, median, 90th-percentile and
latest wave, the median time between consecutive events of a wave, and per
XCD the median key-loop end and the last wave end; plus the launch's span
against HIP events around it.

The timeline build gives the same output bits as libmgqa.so (the marks move
no arithmetic; the GPU tests check it) but its register allocation differs a
little, so its durations are close to, not equal to, the library's.

--check fails (exit status 1) unless every wave of every launch left a
record with non-decreasing event times; --save-output writes the output of
one more call on the first input copy (the seeded inputs; numpy, storage
dtype) for a bit comparison.
"""
from __future__ import annotations

import argparse
import ctypes
import sys
import time

import numpy as np

from . import _lib, synth

TICK_US = 0.01                   # the real-time counter runs at 100 MHz
LLC_BYTES = 256 * 1024 * 1024    # MI355X last-level (Infinity) cache

# Event names per kernel (include/mgqa_timeline.h); None: not used.
EVENTS = {
    "splitkv_kernel": ["start", "Q + first tile requested", "first tile in LDS", "key loop done",
                       "wave states merged, written", "partial stores complete", "arrival counted",
                       "last arrival: splits merged, written"],
    "encoder_kernel": ["start", "K, V requested", "score products issued", "probabilities done",
                       "P.V products issued", "wave states in LDS", "merge weights ready", "output written"],
    "prefill_pipe4_kernel": ["start", "block 1: first tiles in LDS", "block 1: key loop done",
                             "block 1: rows written", "block 2: first tiles in LDS", "block 2: key loop done",
                             "block 2: rows written", "end"],
    "prefill_kernel": ["start", "first tile in LDS", "key loop done", None, None, None, None, "rows written"],
}
# The event that ends a wave's key loop, per kernel (per-XCD table).
LOOP_END = {"splitkv_kernel": 3, "encoder_kernel": 4, "prefill_pipe4_kernel": 2, "prefill_kernel": 2}


def kernel_of(plan: dict, d: int) -> tuple[str, int]:
    """(kernel name, waves per workgroup) of a plan, as the library dispatches."""
    if plan["path"] == 1:
        return "splitkv_kernel", plan["keys_per_tile"] // 32
    if plan["path"] == 2:
        return "encoder_kernel", 8
    if d == 128:
        return "prefill_pipe4_kernel", 4
    return "prefill_kernel", 8


class Launcher:
    """Device copies of one workload and a C-ABI call per copy."""

    def __init__(self, w: synth.Workload):
        import torch
        from . import accounting
        self.torch, self.w = torch, w
        q, k, v = synth.draw_qkv(w)

        def dev(a):
            if w.dtype == "bf16":
                return torch.from_numpy(a.view("int16")).view(torch.bfloat16).cuda()
            return torch.from_numpy(a).cuda()

        touched = accounting.workload_work(w)["bytes"]
        copies = max(3, min(32, -(-2 * LLC_BYTES // max(touched, 1))))
        base = [dev(a) for a in (q, k, v)]
        self.sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
        self.outs = [torch.empty_like(base[0]) for _ in range(copies)]
        self.ws_bytes = _lib.attn_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window)
        self.ws = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device="cuda")
        self.stream = torch.cuda.current_stream().cuda_stream
        dtype_code = _lib.MGQA_BF16 if w.dtype == "bf16" else _lib.MGQA_FP16
        # Arguments marshalled once, so that a call reaches the launch quickly.
        self.fn = _lib.load().attn_fwd_ex
        self.args = [(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(), w.B, w.Hq, w.Hkv, w.Lq, w.Lkv,
                      w.d, int(w.causal), w.window, ctypes.c_float(w.softcap), dtype_code,
                      self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes, self.stream)
                     for (tq, tk, tv), to in zip(self.sets, self.outs)]

    def call(self, i: int) -> None:
        rc = self.fn(*self.args[i % len(self.args)])
        if rc != 0:
            raise RuntimeError(f"attn_fwd_ex failed: {_lib.error_string(rc)}")


def read_records(n_waves: int, events: int) -> np.ndarray:
    """The first n_waves records, shape [n_waves, events + 1] (uint64)."""
    buf = np.zeros((n_waves, events + 1), dtype=np.uint64)
    rc = _lib.attn_timeline_read(buf.ctypes.data, buf.size)
    if rc != 0:
        raise RuntimeError(f"attn_timeline_read: {_lib.error_string(rc)}")
    return buf


def check_records(rec: np.ndarray) -> list[str]:
    """Problems with one launch's records: a wave without a record, or event
    times that decrease along a wave."""
    bad = []
    valid = (rec[:, 0] & np.uint64(1)) == 1
    if not valid.all():
        bad.append(f"{int((~valid).sum())} of {len(rec)} waves left no record")
    t = rec[valid, 1:].astype(np.int64)
    if (t[:, 0] == 0).any():
        bad.append("a wave has no start time")
    for i, row in enumerate(t):
        seen = row[row > 0]
        if (np.diff(seen) < 0).any():
            bad.append(f"wave {i}: event times decrease: {row.tolist()}")
            break
    return bad


def summarise(rec: np.ndarray, kernel: str) -> dict:
    """Statistics of one launch, in µs from the first wave's start."""
    names = EVENTS[kernel]
    valid = (rec[:, 0] & np.uint64(1)) == 1
    rec = rec[valid]
    xcc = ((rec[:, 0] >> np.uint64(4)) & np.uint64(0xF)).astype(np.int64)
    t = rec[:, 1:].astype(np.int64)
    reached = t > 0
    t0 = t[:, 0].min()
    rel = np.where(reached, (t - t0) * TICK_US, np.nan)
    out = {"waves": int(len(rec)), "events": [], "phases": [], "xcd": []}
    for e, name in enumerate(names):
        if name is None or not reached[:, e].any():
            continue
        col = rel[reached[:, e], e]
        out["events"].append({"event": e, "name": name, "waves": int(len(col)),
                              "min": float(col.min()), "median": float(np.median(col)),
                              "p90": float(np.percentile(col, 90)), "max": float(col.max())})
    # Time from each event to the next one the same wave reached.
    steps: dict = {}
    for row, hit in zip(t, reached):
        ev = np.flatnonzero(hit)
        for a_i, b_i in zip(ev, ev[1:]):
            steps.setdefault((int(a_i), int(b_i)), []).append((row[b_i] - row[a_i]) * TICK_US)
    for (a_i, b_i), dts in sorted(steps.items()):
        dt = np.array(dts)
        out["phases"].append({"from": names[a_i], "to": names[b_i], "waves": int(len(dt)),
                              "median": float(np.median(dt)), "p90": float(np.percentile(dt, 90))})
    last = np.nanmax(rel, axis=1)
    out["span"] = float(np.nanmax(last))
    le = LOOP_END[kernel]
    for x in sorted(set(xcc.tolist())):
        sel = xcc == x
        loop = rel[sel & reached[:, le], le]
        out["xcd"].append({"xcd": int(x), "waves": int(sel.sum()),
                           "loop_end_median": float(np.median(loop)) if len(loop) else float("nan"),
                           "last_end": float(np.nanmax(last[sel]))})
    return out


def markdown(w: synth.Workload, kernel: str, plan: dict, waves_per_wg: int, runs: list) -> str:
    lines = [f"Workload `{w.name}` ({w.describe()}), kernel `{kernel}`, {plan['workgroups']} workgroups of "
             f"{waves_per_wg} waves; times in µs from the first wave's start (100 MHz counter).", ""]
    xcds = sorted({x["xcd"] for _, s in runs for x in s["xcd"]})
    lines.append("| launch | HIP events µs | span of the records µs | " +
                 " | ".join(f"XCD {x} loop end / last end" for x in xcds) + " |")
    lines.append("|---" * (3 + len(xcds)) + "|")
    for i, (ev_us, s) in enumerate(runs):
        by = {x["xcd"]: x for x in s["xcd"]}
        cells = " | ".join(f"{by[x]['loop_end_median']:.2f} / {by[x]['last_end']:.2f}" if x in by else "–"
                           for x in xcds)
        lines.append(f"| {i} | {ev_us:.2f} | {s['span']:.2f} | {cells} |")
    last = runs[-1][1]
    lines += ["", f"Events of launch {len(runs) - 1} ({last['waves']} waves):", "",
              "| event | waves | earliest | median | 90th pct | latest |", "|---|---|---|---|---|---|"]
    for e in last["events"]:
        lines.append(f"| {e['event']} {e['name']} | {e['waves']} | {e['min']:.2f} | {e['median']:.2f} | "
                     f"{e['p90']:.2f} | {e['max']:.2f} |")
    lines += ["", "Per wave, from one event to the next (median and 90th percentile over the waves, "
              f"launch {len(runs) - 1}):", "", "| from | to | waves | median | 90th pct |", "|---|---|---|---|---|"]
    for p in last["phases"]:
        lines.append(f"| {p['from']} | {p['to']} | {p['waves']} | {p['median']:.2f} | {p['p90']:.2f} |")
    return "\n".join(lines) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("workload")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=20, help="untimed calls before each recorded launch")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="untimed calls before the first launch, back to back, for at least this long "
                         "(the GPU clocks ramp up under load)")
    ap.add_argument("--check", action="store_true")
    ap.add_argument("--save-output", default=None)
    ap.add_argument("--markdown", default=None)
    args = ap.parse_args(argv)

    w = synth.WORKLOADS.get(args.workload) or synth.NEXT_WORKLOADS.get(args.workload)
    if w is None:
        print(f"unknown workload {args.workload}", file=sys.stderr)
        return 2
    _lib.use_timeline_build()
    import torch
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        return 2
    events, max_waves = _lib.attn_timeline_layout()
    rc, plan = _lib.attn_plan(w.B, w.Hq, w.Hkv, w.Lq, w.Lkv, w.d, int(w.causal), w.window, w.softcap,
                              _lib.MGQA_BF16 if w.dtype == "bf16" else _lib.MGQA_FP16)
    if rc != 0:
        raise RuntimeError(f"attn_plan: {_lib.error_string(rc)}")
    kernel, wpw = kernel_of(plan, w.d)
    n_waves = plan["workgroups"] * wpw
    if n_waves > max_waves:
        print(f"{n_waves} waves exceed the {max_waves} records of the timeline build", file=sys.stderr)
        return 2
    run = Launcher(w)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Records are summarised after the last launch: host work between the
    # launches would let the GPU clocks drop before the next one.
    recs, times, problems = [], [], []
    i = 0
    t_end = time.perf_counter() + args.warmup_seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            run.call(i)
            i += 1
        torch.cuda.synchronize()
    for launch in range(args.launches):
        for _ in range(args.warmup):
            run.call(i)
            i += 1
        torch.cuda.synchronize()
        rc = _lib.attn_timeline_clear(run.stream)
        if rc != 0:
            raise RuntimeError(f"attn_timeline_clear: {_lib.error_string(rc)}")
        torch.cuda.synchronize()
        start.record()
        run.call(i)
        end.record()
        torch.cuda.synchronize()
        recs.append(read_records(n_waves, events))
        times.append(start.elapsed_time(end) * 1e3)
        i += 1
    runs = []
    for launch, (rec, ev_us) in enumerate(zip(recs, times)):
        problems += [f"launch {launch}: {p}" for p in check_records(rec)]
        s = summarise(rec, kernel)
        runs.append((ev_us, s))
        print(f"launch {launch}: HIP events {ev_us:.2f} us, span {s['span']:.2f} us, {s['waves']} waves", flush=True)
    if args.save_output:
        run.call(0)
        torch.cuda.synchronize()
        out = run.outs[0].cpu()
        arr = out.view(torch.int16).numpy().view(np.uint16) if w.dtype == "bf16" else out.numpy()
        np.save(args.save_output, arr)
    text = markdown(w, kernel, plan, wpw, runs)
    print(text, flush=True)
    if args.markdown:
        with open(args.markdown, "w") as f:
            f.write(text)
    if args.check and problems:
        print("\n".join(problems), file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
