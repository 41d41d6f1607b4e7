#!/usr/bin/env python3
"""Benchmark of the hyper-connection hot path on one MI355X.

One step = the whole per-sublayer hot path over one batch: the fused
hc_mixes + split/Sinkhorn + hc_pre call, then hc_post, on the large-prefill
workload (B=8, T=8192, hc=4, d=5120: 65,536 tokens, a 2.7 GB bf16 residual)
with every input resident in HBM before timing starts.  Prints one JSON
line: whole-step tokens/s, the dominant kernel's achieved HBM bandwidth
against the 8 TB/s peak (``roofline``), and the fp64 CPU oracle timed on the
host (``cpu_baseline``).

    python bench.py [--steps K] [--warmup W] [--workload large|prefill|decode]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E peak, GB/s

PROFILE_DIR = os.path.join(ROOT, "profiles")


def algorithmic_bytes(n: int, d: int):
    """Minimum HBM bytes per launch: every input read once, every output
    written once.  fused: R + h + pre/post/comb (+ the weights, once per
    launch); hc_post: R + x + post/comb + R'."""
    hc = 4
    fused = n * (hc * d * 2 + d * 2 + (hc + hc + hc * hc) * 4) + 24 * hc * d * 4 + 27 * 4
    post = n * (hc * d * 2 + d * 2 + (hc + hc * hc) * 4 + hc * d * 2)
    return fused, post


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hyper_connection_residual_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, n: int, d: int):
    """HBM bytes per launch of ``kernel`` from the committed counter summary,
    or None when there is none for this workload or the kernels changed
    since it was taken."""
    path = os.path.join(PROFILE_DIR, "hbm_traffic_%s_n%d_d%d.json" % (kernel, n, d))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large", choices=["large", "prefill", "decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32768, help="tokens the oracle is timed on")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path is per-token independent and "
              "shards by tokens with no exchange; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import hyper_connection_residual_02_amd as hcl
    from hyper_connection_residual_02_amd import inputs as hin

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hcl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = hin.WORKLOADS[args.workload]
    n, d = w.n, w.d
    t = hin.make_inputs(w, dev)
    R, x, W, s, b = t["R"], t["x"], t["W"], t["scale"], t["base"]
    ws = hcl.Workspace()
    outs = dict(h=torch.empty(w.B, w.T, d, dtype=torch.bfloat16, device=dev),
                pre=torch.empty(w.B, w.T, 4, device=dev),
                post=torch.empty(w.B, w.T, 4, device=dev),
                comb=torch.empty(w.B, w.T, 4, 4, device=dev))
    Rout = torch.empty_like(R)

    def fused():
        hcl.hc_fused_mix_pre(R, W, s, b, sinkhorn_iters=w.iters, hc_eps=w.hc_eps,
                             norm_eps=w.norm_eps, workspace=ws, out=outs)

    def post():
        hcl.hc_post(x, R, outs["post"], outs["comb"], out=Rout)

    def step():
        fused()
        post()

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, synchronised on both sides
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps

    # ---- per-kernel launch durations (HIP events on the launch stream)
    def time_each(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, z in evs:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        v = np.array([a.elapsed_time(z) for a, z in evs]) * 1e3     # us
        return float(v.mean()), float(np.median(v)), float(v.min())

    reps = max(args.steps, 10)
    f_mean, f_med, f_min = time_each(fused, reps)
    p_mean, p_med, p_min = time_each(post, reps)
    fb, pb = algorithmic_bytes(n, d)
    f_gbs = fb / (f_mean * 1e-6) / 1e9
    p_gbs = pb / (p_mean * 1e-6) / 1e9

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if p_mean >= f_mean:
        dom = dict(name="hc_post", kernel="k_post", us=p_mean, bytes=pb, gbs=p_gbs)
    else:
        dom = dict(name="hc_fused_mix_pre", kernel="k_coop", us=f_mean, bytes=fb, gbs=f_gbs)
    traffic = measured_traffic(dom["kernel"], n, d)

    # ---- CPU baseline: the fp64 oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        k = min(args.cpu_sample, n)
        Rb = hin.bits(R.reshape(n, 4, d)[:k])
        xb = hin.bits(x.reshape(n, d)[:k])
        Wn, sn, bn = W.cpu().numpy(), s.cpu().numpy(), b.cpu().numpy()
        c0 = time.perf_counter()
        _, _, oq, oc, _ = oracle.fused(Rb, Wn, sn, bn, w.iters, w.hc_eps, w.norm_eps)
        oracle.post(xb, Rb, oq, oc)
        csec = time.perf_counter() - c0
        cpu = {"value": k / csec, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "first %d of %d tokens of the same inputs (fused mix+Sinkhorn+pre, then "
                         "hc_post), %.1f s" % (k, n, csec)}

    tok_s = n / (ms_step * 1e-3)
    line = {
        "metric": "tokens/s + achieved HBM GB/s (% of peak), fused hc mix+pre and hc_post, d=5120",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) residual and sublayer output, N(0,0.007) weights)",
        "config": {"workload": "%s: B=%d T=%d hc=4 d=%d (%d tokens), sinkhorn_iters=%d"
                               % (w.name, w.B, w.T, d, n, w.iters),
                   "tokens": n, "d": d, "hc": 4, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dom["name"], "achieved": round(dom["gbs"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom["gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": dom["bytes"],
                     "avg_launch_us": round(dom["us"], 2)},
        "kernels": {
            "hc_fused_mix_pre": {"avg_us": round(f_mean, 2), "median_us": round(f_med, 2),
                                 "min_us": round(f_min, 2), "GB/s": round(f_gbs, 1),
                                 "frac_of_peak": round(f_gbs / HBM_PEAK_GBS, 4),
                                 "tokens/s": round(n / (f_mean * 1e-6), 1), "bytes": fb},
            "hc_post": {"avg_us": round(p_mean, 2), "median_us": round(p_med, 2), "min_us": round(p_min, 2),
                        "GB/s": round(p_gbs, 1), "frac_of_peak": round(p_gbs / HBM_PEAK_GBS, 4),
                        "tokens/s": round(n / (p_mean * 1e-6), 1), "bytes": pb},
        },
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
