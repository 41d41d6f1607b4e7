"""The phase-tracing build (libhc_trace.so, hc_phase_trace) on the GPU.

The traced library must compute exactly what libhc.so computes: the fused
call and the sublayer-boundary call run through both builds (each in a
process of its own, since the binding loads one library per process) and
every output is compared bitwise.  Its tables must describe the launch: one
entry per workgroup of the persistent kernel, each with the round loop's
tick count (rounds of the workgroup's token group + 2) and phase totals that
add up to no more than the loop's duration, and clock stamps in order.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import hyper_connection_residual_02_amd as hcl

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, %(root)r)
import hyper_connection_residual_02_amd as hcl
from hyper_connection_residual_02_amd import inputs as hin
if %(trace)r:
    hcl.use_library(hcl.trace_library_path())
w = hin.Workload("phase", 1, %(n)d, 4, 5120, 0.007, 0.5, 2.0, 1.0)
t = hin.make_inputs(w, "cuda", seed=11)
h, pre, post, comb, mixes = hcl.hc_fused_mix_pre(t["R"], t["W"], t["scale"], t["base"], want_pre=True,
                                                 want_mixes=True)
res = dict(h=hin.bits(h), pre=pre.cpu().numpy(), post=post.cpu().numpy(), comb=comb.cpu().numpy(),
           mixes=mixes.cpu().numpy())
if %(trace)r:
    res["trace_fused"] = hcl.phase_trace(1024 * 60)
nxt = hin.make_inputs(w, "cuda", seed=12)
R2, h2, pre2, post2, comb2, mixes2 = hcl.hc_post_mix_pre(t["x"], t["R"], post, comb, nxt["W"], nxt["scale"],
                                                         nxt["base"], want_pre=True, want_mixes=True)
torch.cuda.synchronize()
res.update(h2=hin.bits(h2), pre2=pre2.cpu().numpy(), post2=post2.cpu().numpy(), comb2=comb2.cpu().numpy(),
           mixes2=mixes2.cpu().numpy(), R2=hin.bits(R2))
if %(trace)r:
    res["trace_boundary"] = hcl.phase_trace(1024 * 60)
np.savez(%(out)r, **res)
"""


def _run(trace, n, out):
    code = CHILD % dict(root=ROOT, trace=trace, n=n, out=out)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]


def test_traced_build_is_bitwise_the_library_and_its_tables_describe_the_launch(tmp_path):
    if not os.path.exists(hcl.trace_library_path()):
        pytest.skip("libhc_trace.so not built (python -m hyper_connection_residual_02_amd.build --phase-trace)")
    n = 4100                                     # persistent path, a ragged last round
    _run(False, n, str(tmp_path / "plain.npz"))
    _run(True, n, str(tmp_path / "trace.npz"))
    a, b = np.load(tmp_path / "plain.npz"), np.load(tmp_path / "trace.npz")
    for k in a.files:
        assert np.array_equal(a[k], b[k]), k
    rounds = (n + 31) // 32
    for key in ("trace_fused", "trace_boundary"):
        assert b[key].size == 1024 * 60, (key, b[key].size)
        tr = b[key][:1024 * 56].reshape(-1, 8, 7)
        ts = b[key][1024 * 56:].reshape(-1, 4)[:256].astype(np.int64)
        # every workgroup's stamps in order: entry <= start-up done <= loop start <= end
        assert np.all(np.diff(ts, axis=1) >= 0), key
        assert np.all(ts[:, 3] - ts[:, 0] < 100_000_000), key
        ran = tr[:, 0, 6] > 0
        assert ran.sum() == 256, (key, int(ran.sum()))       # 8 token groups x 32 members at d = 5120
        assert np.all(ran[:256]) and not ran[256:].any(), key
        tr = tr[:256]
        # workgroup b is member b / 8 of token group g = b % 8, which has
        # ceil((rounds - g) / 8) rounds; the loop runs two ticks more
        for blk in range(256):
            g = blk % 8
            nr = (rounds - g + 7) // 8
            assert np.all(tr[blk, :, 6] == nr + 2), (key, blk, tr[blk, :, 6])
        # phase totals are 100 MHz ticks: each wave's sum stays within the
        # call's time on the device (far less than a second) and is positive
        tot = tr[:, :, :6].sum(axis=2)
        assert np.all(tot > 0) and np.all(tot < 100_000_000), key
