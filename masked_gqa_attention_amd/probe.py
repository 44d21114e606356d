"""Throughput probes of one MI355X: the rates the attention kernels' rooflines
rest on (include/mgqa_probe.h, libmgqa_probe.so).

    python -m masked_gqa_attention_amd.probe [--quick] [--markdown PATH]

Measures, each from HIP events around back-to-back launches on one stream:
* the issue cost of one bf16 16x16x32 matrix-core product, one v_exp_f32,
  one v_rcp_f32 and one v_mul_f32 per SIMD (independent chains, with two and
  eight waves per SIMD), and of a product interleaved with one exp or one mul;
* one step of the head-size-128 prefill with a softcap (34 products, 48
  transcendental and 48 plain vector operations per wave, a barrier;
  one, two and four workgroups of four waves per CU): matrix work alone,
  vector work alone, both;
* the streaming read rate of device buffers of the 4:1 decode's size
  (268.6 MB) and of 1 GiB, with plain and with non-temporal loads, with
  three grid sizes.
Prints a markdown report.  --quick: small sizes (a smoke check, not a
measurement).
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import torch  # noqa: F401  (loads the HIP runtime first, as _lib does)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmgqa_probe.so")

# include/mgqa_probe.h
PROBE_MFMA, PROBE_EXP, PROBE_RCP, PROBE_MUL = 0, 1, 2, 3
PROBE_MFMA_EXP, PROBE_MFMA_MUL = 4, 5
PROBE_STEP_MFMA, PROBE_STEP_VEC, PROBE_STEP_BOTH = 6, 7, 8
EXPORTS = ("probe_alu", "probe_read")

# Per wave and iteration: (matrix products, vector instructions) of each kind.
WORK = {
    PROBE_MFMA: (8, 0), PROBE_EXP: (0, 8), PROBE_RCP: (0, 8), PROBE_MUL: (0, 8),
    PROBE_MFMA_EXP: (8, 8), PROBE_MFMA_MUL: (8, 8),
    PROBE_STEP_MFMA: (34, 0), PROBE_STEP_VEC: (0, 96), PROBE_STEP_BOTH: (34, 96),
}
MFMA_FLOPS = 16 * 16 * 32 * 2
CUS, SIMDS_PER_CU = 256, 4

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m masked_gqa_attention_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i = ctypes.c_void_p, ctypes.c_int
        lib.probe_alu.argtypes = [i, i, i, i, vp, vp]
        lib.probe_alu.restype = i
        lib.probe_read.argtypes = [vp, ctypes.c_size_t, i, i, vp, vp]
        lib.probe_read.restype = i
        _lib = lib
    return _lib


def _timed(launch, reps: int) -> float:
    """Milliseconds per launch over `reps` back-to-back launches (one untimed first)."""
    launch()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        launch()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / reps


def run_alu(kind: int, workgroups: int, waves: int, iters: int, reps: int = 5) -> dict:
    """One ALU probe; ns per instruction per SIMD assumes every SIMD holds
    the same number of the launch's waves."""
    lib = load()
    sink = torch.empty(workgroups * waves * 64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.probe_alu(kind, workgroups, waves, iters, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe_alu({kind}) failed: {rc}")

    ms = _timed(launch, reps)
    mfma, vec = WORK[kind]
    wave_iters = workgroups * waves * iters
    simds = CUS * SIMDS_PER_CU
    out = {"kind": kind, "workgroups": workgroups, "waves": waves, "iters": iters, "ms": ms,
           "ns_per_iter_per_simd": ms * 1e6 * simds / wave_iters,
           "finite": bool(torch.isfinite(sink.view(torch.float32)).all().item())}
    if mfma:
        out["tflops"] = wave_iters * mfma * MFMA_FLOPS / (ms * 1e-3) / 1e12
        out["ns_per_mfma_per_simd"] = ms * 1e6 * simds / (wave_iters * mfma)
    if vec:
        out["ns_per_vec_per_simd"] = ms * 1e6 * simds / (wave_iters * vec)
        out["lane_gops"] = wave_iters * vec * 64 / (ms * 1e-3) / 1e9
    return out


def run_read(nbytes: int, workgroups: int, nontemporal: bool = False, reps: int = 5) -> dict:
    lib = load()
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    sink = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.probe_read(buf.data_ptr(), nbytes, workgroups, int(nontemporal), sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"probe_read failed: {rc}")

    ms = _timed(launch, reps)
    return {"bytes": nbytes, "workgroups": workgroups, "nontemporal": nontemporal, "ms": ms,
            "gbs": nbytes / (ms * 1e-3) / 1e9}


NAMES = {PROBE_MFMA: "bf16 16x16x32 products", PROBE_EXP: "v_exp_f32", PROBE_RCP: "v_rcp_f32",
         PROBE_MUL: "v_mul_f32", PROBE_MFMA_EXP: "product + v_exp_f32", PROBE_MFMA_MUL: "product + v_mul_f32",
         PROBE_STEP_MFMA: "prefill step: matrix work", PROBE_STEP_VEC: "prefill step: vector work",
         PROBE_STEP_BOTH: "prefill step: both"}


def measure(quick: bool = False) -> dict:
    scale = 0.02 if quick else 1.0
    it = lambda n: max(1, int(n * scale))  # noqa: E731
    res = {"alu": [], "step": [], "read": None}
    for waves_per_simd in (2, 8):
        wgs = CUS * waves_per_simd  # workgroups of four waves, one per SIMD
        for kind, iters in ((PROBE_MFMA, 4000), (PROBE_EXP, 4000), (PROBE_RCP, 4000), (PROBE_MUL, 8000),
                            (PROBE_MFMA_EXP, 4000), (PROBE_MFMA_MUL, 4000)):
            res["alu"].append(run_alu(kind, wgs, 4, it(iters // waves_per_simd * 2)))
    for per_cu in (1, 2, 4):
        # Workgroups of four waves (one per SIMD); the prefill runs two per CU.
        for kind in (PROBE_STEP_MFMA, PROBE_STEP_VEC, PROBE_STEP_BOTH):
            r = run_alu(kind, per_cu * CUS, 4, it(2000))
            r["per_cu"] = per_cu
            res["step"].append(r)
    res["read"] = []
    for nbytes in ((1 << 24,) if quick else (268566528, 1 << 30)):
        for nt in (False, True):
            for wgs in (CUS * 4, CUS * 8, CUS * 16):
                res["read"].append(run_read(nbytes, wgs, nt))
    return res


def markdown(res: dict, command: str) -> str:
    props = torch.cuda.get_device_properties(0)
    lines = ["# Throughput probes (libmgqa_probe.so)", "",
             "Command (repo root, one MI355X, after `python -m masked_gqa_attention_amd.build`):", "",
             f"    {command}", "",
             f"Device: {props.name}, {props.multi_processor_count} compute units, "
             f"{getattr(props, 'gcnArchName', '?')}.  Kernels and their work per wave and iteration: "
             "`include/mgqa_probe.h`.  Times from HIP events around 5 back-to-back launches; "
             "per-SIMD figures assume the launch's waves spread evenly over the 1024 SIMDs.", "",
             "## Instruction issue cost (independent chains)", "",
             "| probe | waves per SIMD | ms per launch | ns per product per SIMD | ns per vector op per SIMD "
             "| TFLOP/s | lane Gop/s |",
             "|---|---|---|---|---|---|---|"]
    def cell(r, key, fmt):
        return format(r[key], fmt) if key in r else "—"

    for r in res["alu"]:
        wps = r["workgroups"] // CUS
        lines.append(f"| {NAMES[r['kind']]} | {wps} | {r['ms']:.3f} | {cell(r, 'ns_per_mfma_per_simd', '.2f')} | "
                     f"{cell(r, 'ns_per_vec_per_simd', '.2f')} | {cell(r, 'tflops', '.1f')} | "
                     f"{cell(r, 'lane_gops', '.0f')} |")
    lines += ["", "## One prefill step (workgroups of four waves, a barrier per step)", "",
              "The prefill kernel runs two workgroups per CU.", "",
              "| probe | workgroups per CU | ms per launch | steps | ns per step of a CU (all its workgroups) "
              "| ns per workgroup step |", "|---|---|---|---|---|---|"]
    for r in res["step"]:
        per_step = r["ms"] * 1e6 / r["iters"]
        lines.append(f"| {NAMES[r['kind']]} | {r['per_cu']} | {r['ms']:.3f} | {r['iters']} | {per_step:.0f} "
                     f"| {per_step / r['per_cu']:.0f} |")
    lines += ["", "## Streaming read (16-byte loads, workgroups of 256 threads)", "",
              "| bytes | loads | workgroups | µs | GB/s | % of 8 TB/s |", "|---|---|---|---|---|---|"]
    for rd in res["read"]:
        kind = "non-temporal" if rd["nontemporal"] else "plain"
        lines.append(f"| {rd['bytes']} | {kind} | {rd['workgroups']} | {rd['ms'] * 1e3:.1f} | {rd['gbs']:.0f} "
                     f"| {rd['gbs'] / 8000 * 100:.1f} |")
    lines.append("")
    return "\n".join(lines)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--quick", action="store_true")
    ap.add_argument("--markdown", default=None)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("no GPU", file=sys.stderr)
        return 2
    res = measure(quick=args.quick)
    cmd = "python -u -m masked_gqa_attention_amd.probe" + (" --quick" if args.quick else "") + \
        (f" --markdown {args.markdown}" if args.markdown else "")
    text = markdown(res, cmd)
    print(text, flush=True)
    if args.markdown:
        with open(args.markdown, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
