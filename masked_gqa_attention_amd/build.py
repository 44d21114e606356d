"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m masked_gqa_attention_amd.build [--verbose]

Every HIP source is compiled for gfx950 only, with packed fp32 instructions
disabled and matrix-core accumulators in architectural registers, and
linked into masked_gqa_attention_amd/libmgqa.so next to this file.  The
same sources with the kernels compiled under MGQA_TIMELINE give
libmgqa_timeline.so, the measurement build with per-wave timestamps
(include/mgqa_timeline.h), and mgqa_probe.hip gives libmgqa_probe.so, the
throughput probes (include/mgqa_probe.h).  The build always recompiles (it
is the "does it build" check).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmgqa.so")
OUT_TIMELINE = os.path.join(PKG, "libmgqa_timeline.so")
OUT_PROBE = os.path.join(PKG, "libmgqa_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["mgqa_api.cpp", "mgqa_kernels.hip", "mgqa_cache.hip"]
TIMELINE_SOURCE = "mgqa_kernels.hip"  # the only source with timeline marks
PROBE_SOURCE = "mgqa_probe.hip"

ARCH = "gfx950"
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core instructions take their accumulators in architectural
    # registers: with the heuristic choice the split-KV kernels kept the
    # accumulators in accumulation registers and copied them back and forth
    # on every key tile (same results, 14% slower on the 729-token encoder).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmgqa.so")
    return path


def _compile(src: str, verbose: bool, timeline: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + (".timeline.o" if timeline else ".o"))
    defs = ["-DMGQA_TIMELINE"] if timeline else []
    cmd = [hipcc(), *COMMON, *defs, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Builds libmgqa.so, libmgqa_timeline.so and libmgqa_probe.so; returns
    the first one's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + [(TIMELINE_SOURCE, True), (PROBE_SOURCE, False)]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], verbose, j[1]), jobs))
    plain = objs[:len(SOURCES)]
    timeline = [objs[len(SOURCES)] if s == TIMELINE_SOURCE else o for s, o in zip(SOURCES, plain)]
    _link(plain, OUT, verbose)
    _link(timeline, OUT_TIMELINE, verbose)
    _link([objs[-1]], OUT_PROBE, verbose)
    return OUT


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    out = build(verbose=args.verbose)
    print(out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
