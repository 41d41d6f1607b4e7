"""Build libhc (HIP, gfx950) in-tree: hyper_connection_residual_02_amd/libhc.so.

Usage: python -m hyper_connection_residual_02_amd.build [--phase-trace]

--phase-trace also builds libhc_trace.so: the same library with the
persistent projection kernel's phase tracing compiled in (hc_phase_trace;
bench.py --phases).  It is a diagnostic build, slower than libhc.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libhc.so")
OUT_TRACE = os.path.join(PKG, "libhc_trace.so")
BUILD = os.path.join(ROOT, "_build")
TRACED = ["hc_api.hip", "hc_coop.hip"]          # the sources the tracing switch changes
SOURCES = ["hc_api.hip", "hc_stream.hip", "hc_sinkhorn.hip", "hc_coop.hip", "hc_general.hip", "hc_backward.hip",
           "hc_norm.hip", "hc_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-result",
]


def _compile(job) -> str:
    src, trace = job
    obj = os.path.join(BUILD, ("trace_" if trace else "") + os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DHC_PHASE_TRACE"] if trace else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, msgs))
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, out)


def build(verbose: bool = True, phase_trace: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libhc.so in-tree (and,
    with phase_trace, libhc_trace.so)."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in TRACED] if phase_trace else [])
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = dict(zip(jobs, ex.map(_compile, jobs)))
    _link([objs[(src, False)] for src in SOURCES], OUT)
    if verbose:
        print("built", OUT)
    if phase_trace:
        _link([objs[(src, src in TRACED)] for src in SOURCES], OUT_TRACE)
        if verbose:
            print("built", OUT_TRACE)
    return OUT


if __name__ == "__main__":
    build(phase_trace="--phase-trace" in sys.argv[1:])
