"""GPU parity: every libhc entry point against the fp64 CPU oracle.

The GPU side is always called through the C-ABI (via the thin binding);
the oracle is fed the very same input tensors.  Full-size workloads are
checked on every token when the oracle finishes in seconds (tiny, decode,
prefill) and on sampled tokens otherwise (large prefill: 65,536 tokens),
in the launch configuration the benchmark uses.  Tolerances: tests/hc_check.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

import hyper_connection_residual_02_amd as hcl
from hyper_connection_residual_02_amd import inputs as hin
from hc_check import (check_abs, check_bf16_exact, check_bf16_tol, check_mixes, post_terms,
                      pre_terms)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hcl.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _np(t):
    return t.detach().cpu().numpy()


def run_fused(R, W, s, b, iters=20, eps=1e-6, neps=1e-20):
    h, pre, post, comb, mixes = hcl.hc_fused_mix_pre(R, W, s, b, sinkhorn_iters=iters, hc_eps=eps,
                                                     norm_eps=neps, want_pre=True, want_mixes=True)
    torch.cuda.synchronize()
    return h, pre, post, comb, mixes


def compare_fused(orc, R, W, s, b, outs, idx=None, iters=20, eps=1e-6, neps=1e-20, x=None, label=""):
    """Oracle on tokens idx (all when None) vs the GPU outputs of the fused
    call; then hc_post on the GPU coefficients if x is given."""
    h, pre, post, comb, mixes = outs
    hc, d = R.shape[-2], R.shape[-1]
    Rf = R.reshape(-1, hc, d)
    n = Rf.shape[0]
    sel = torch.arange(n, device=R.device) if idx is None else torch.as_tensor(idx, device=R.device)
    Rb = hin.bits(Rf[sel])
    g = {k: _np(v.reshape(n, *v.shape[len(R.shape) - 2:])[sel]) for k, v in
         dict(pre=pre, post=post, comb=comb, mixes=mixes).items()}
    gh = hin.bits(h.reshape(n, d)[sel])
    Wn, sn, bn = _np(W), _np(s), _np(b)
    # end to end: oracle from R
    om = orc.mixes(Rb, Wn, neps)
    op, oq, oc = orc.split_sinkhorn(om, sn, bn, hc, iters, eps)
    oh = orc.pre(Rb, op)
    check_mixes(g["mixes"], om)
    check_abs(g["pre"], op, label + " pre")
    check_abs(g["post"], oq, label + " post")
    check_abs(g["comb"], oc, label + " comb")
    check_bf16_tol(gh, oh, lambda: pre_terms(Rb, op), label + " h end-to-end")
    # isolated: oracle split on the GPU's own mixes; oracle hc_pre on its pre
    ip, iq, ic = orc.split_sinkhorn(g["mixes"].astype(np.float64), sn, bn, hc, iters, eps)
    check_abs(g["pre"], ip, label + " pre (isolated)")
    check_abs(g["post"], iq, label + " post (isolated)")
    check_abs(g["comb"], ic, label + " comb (isolated)")
    check_bf16_exact(gh, orc.pre(Rb, g["pre"].astype(np.float64)), label + " h (isolated)")
    if x is not None:
        Rout = hcl.hc_post(x, R, post, comb)
        torch.cuda.synchronize()
        xb = hin.bits(x.reshape(n, d)[sel])
        go = hin.bits(Rout.reshape(n, hc, d)[sel])
        check_bf16_exact(go, orc.post(xb, Rb, g["post"].astype(np.float64), g["comb"].astype(np.float64)),
                         label + " R' (isolated)")
        check_bf16_tol(go, orc.post(xb, Rb, oq, oc), lambda: post_terms(xb, Rb, oq, oc), label + " R' end-to-end")
    return om


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill"])
def test_fused_and_post_full(orc, name):
    w = hin.WORKLOADS[name]
    t = hin.make_inputs(w, DEV)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"])
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, x=t["x"], label=name)


def test_fused_and_post_large_sampled(orc):
    w = hin.WORKLOADS["large"]
    t = hin.make_inputs(w, DEV)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"])
    idx = hin.sample_tokens(w.n, 160)
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, idx=idx, x=t["x"], label="large")
    # properties that hold at any size: coefficient ranges and column sums on every token
    pre, post, comb = outs[1].reshape(-1, 4), outs[2].reshape(-1, 4), outs[3].reshape(-1, 4, 4)
    assert bool(((pre > 0) & (pre <= 1 + 1e-6 + 1e-7)).all())
    assert bool(((post >= 0) & (post <= 2)).all())
    cs = comb.sum(1)
    assert bool(((1 - cs) >= -2e-7).all()) and bool(((1 - cs) < 1e-4).all())
    assert bool(torch.isfinite(outs[4]).all())
    del t, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [1, 2, 15, 16, 17, 31, 33, 63, 100, 255, 257, 2048, 2049, 4095, 4097])
def test_ragged_token_counts(orc, n):
    w = hin.WORKLOADS["prefill"]
    t = hin.make_inputs(w, DEV, seed=7, n_tokens=n)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"])
    idx = None if n <= 300 else hin.sample_tokens(n, 64)
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, idx=idx, x=t["x"], label="n=%d" % n)


@pytest.mark.parametrize("n", [100, 2100])
@pytest.mark.parametrize("iters,eps", [(1, 1e-6), (20, 0.0), (1, 0.0), (3, 1e-3)])
def test_fused_degenerate_parameters(orc, n, iters, eps):
    # one Sinkhorn step (the softmax and a single column normalisation),
    # eps = 0, and a large eps, on the two-pass (100 tokens) and the
    # persistent path (2,100)
    w = hin.WORKLOADS["prefill"]
    t = hin.make_inputs(w, DEV, seed=83, n_tokens=n)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"], iters=iters, eps=eps)
    idx = None if n <= 300 else hin.sample_tokens(n, 64)
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, idx=idx, iters=iters, eps=eps, x=t["x"],
                  label="n=%d iters=%d eps=%g" % (n, iters, eps))


@pytest.mark.timeout(300)
def test_maximum_size_sampled(orc):
    # 262,144 tokens (B = 32, T = 8192) at d = 5120: a 10.7 GB residual, four
    # times the large prefill, so byte offsets into R, x, h and R' pass 2^33;
    # sampled tokens (the first, the last and random ones) against the oracle
    w = hin.Workload("max", 32, 8192, 4, 5120, 0.007, 0.5, 2.0, 1.0)
    t = hin.make_inputs(w, DEV, seed=71)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"])
    idx = hin.sample_tokens(w.B * w.T, 96)
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, idx=idx, x=t["x"], label="max size")
    del t, outs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [32, 64, 256, 1024, 2048, 3072, 4096, 7168, 8192])
def test_other_widths(orc, d):
    # every k-step count of the projection kernel (d = 32*KS*G), ragged n
    w = hin.Workload("w%d" % d, 1, 77, 4, d, 1.0 / np.sqrt(4 * d), 0.5, 2.0, 1.0)
    t = hin.make_inputs(w, DEV, seed=3)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"])
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, x=t["x"], label="d=%d" % d)


def test_standalone_entry_points_match_fused_bitwise(orc):
    w = hin.WORKLOADS["prefill"]
    t = hin.make_inputs(w, DEV, seed=5, n_tokens=1000)
    h, pre, post, comb, mixes = run_fused(t["R"], t["W"], t["scale"], t["base"])
    m2 = hcl.hc_mixes(t["R"], t["W"])
    p2, q2, c2 = hcl.hc_split_sinkhorn(m2, t["scale"], t["base"])
    h2 = hcl.hc_pre(t["R"], p2)
    torch.cuda.synchronize()
    assert torch.equal(m2, mixes)
    assert torch.equal(p2, pre) and torch.equal(q2, post) and torch.equal(c2, comb)
    assert torch.equal(h2, h)


def test_split_standalone_vs_oracle(orc):
    # random mixes with steep scales: the Sinkhorn path on its own
    rng = np.random.default_rng(21)
    n = 5000
    m = (rng.standard_normal((n, 24)) * 2).astype(np.float32)
    for scale in ([1.0, 1.0, 1.0], [0.5, 2.0, 20.0], [2.0, 0.5, 8.0]):
        s = np.array(scale, np.float32)
        b = (rng.standard_normal(24) * 2).astype(np.float32)
        gp, gq, gc = hcl.hc_split_sinkhorn(torch.from_numpy(m).to(DEV), torch.from_numpy(s).to(DEV),
                                           torch.from_numpy(b).to(DEV))
        torch.cuda.synchronize()
        op, oq, oc = orc.split_sinkhorn(m.astype(np.float64), s, b)
        check_abs(_np(gp), op, "pre")
        check_abs(_np(gq), oq, "post")
        check_abs(_np(gc), oc, "comb")
    for iters in (1, 2, 7):
        s = np.array([1.0, 1.0, 3.0], np.float32)
        gp, gq, gc = hcl.hc_split_sinkhorn(torch.from_numpy(m).to(DEV), torch.from_numpy(s).to(DEV),
                                           torch.from_numpy(b).to(DEV), sinkhorn_iters=iters)
        torch.cuda.synchronize()
        check_abs(_np(gc), orc.split_sinkhorn(m.astype(np.float64), s, b, iters=iters)[2], "comb it=%d" % iters)


def test_split_closed_forms():
    # W = 0 gives zero mixes: uniform comb (1 - eps)/4, pre = sigmoid(b) + eps, post = 2 sigmoid(b)
    n = 64
    m = torch.zeros(n, 24, device=DEV)
    b = torch.zeros(24, device=DEV)
    b[8:] = 0.7
    p, q, c = hcl.hc_split_sinkhorn(m, torch.tensor([1.0, 1.0, 4.0], device=DEV), b)
    torch.cuda.synchronize()
    assert torch.allclose(c, torch.full_like(c, (1 - 1e-6) / 4), rtol=0, atol=2e-7)
    assert torch.allclose(p, torch.full_like(p, 0.5 + 1e-6), rtol=0, atol=1e-7)
    assert torch.equal(q, torch.ones_like(q))


def test_post_special_cases_bitwise():
    w = hin.WORKLOADS["decode"]
    t = hin.make_inputs(w, DEV, seed=11)
    R, x = t["R"], t["x"]
    n = w.n
    zeros = torch.zeros(w.B, w.T, 4, device=DEV)
    eye = torch.eye(4, device=DEV).expand(w.B, w.T, 4, 4).contiguous()
    assert torch.equal(hcl.hc_post(x, R, zeros, eye), R)
    out = hcl.hc_post(x, R, torch.ones_like(zeros), torch.zeros_like(eye))
    assert all(torch.equal(out[:, :, k], x) for k in range(4))
    for j, k in [(0, 2), (3, 1), (2, 2)]:
        cb = torch.zeros_like(eye)
        cb[..., j, k] = 1.0
        out = hcl.hc_post(x, R, zeros, cb)
        assert torch.equal(out[:, :, k], R[:, :, j])
    # one-hot pre picks a stream
    for k in range(4):
        p = torch.zeros(w.B, w.T, 4, device=DEV)
        p[..., k] = 1.0
        assert torch.equal(hcl.hc_pre(R, p), R[:, :, k])
    torch.cuda.synchronize()
    del n


def test_post_in_place_matches_out_of_place():
    w = hin.WORKLOADS["prefill"]
    t = hin.make_inputs(w, DEV, seed=13, n_tokens=777)
    _, _, post, comb, _ = run_fused(t["R"], t["W"], t["scale"], t["base"])
    ref = hcl.hc_post(t["x"], t["R"], post, comb)
    R2 = t["R"].clone()
    hcl.hc_post(t["x"], R2, post, comb, out=R2)
    torch.cuda.synchronize()
    assert torch.equal(R2, ref)


def test_determinism_and_batch_invariance():
    w = hin.WORKLOADS["prefill"]
    t = hin.make_inputs(w, DEV, seed=17)
    a = run_fused(t["R"], t["W"], t["scale"], t["base"])
    b = run_fused(t["R"], t["W"], t["scale"], t["base"])
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    # a token's results do not depend on which other tokens share the call
    sub = t["R"][:, 1000:1100].contiguous()
    c = run_fused(sub, t["W"], t["scale"], t["base"])
    for u, v in zip(a, c):
        assert torch.equal(u[:, 1000:1100], v)


TWO_PASS_MAX_N = 2048   # calls of at most this many tokens take the two-pass path


@pytest.mark.parametrize("d", [256, 1024, 2048, 3072, 4096, 5120])
def test_two_pass_and_persistent_paths_agree_bitwise(d):
    # A call of at most 2,048 tokens (at the widths the wave-specialised
    # kernel serves) runs as two ordinary launches: per-member partial sums,
    # then the reduction, split and h.  A longer call runs the persistent
    # kernel.  A token gets bitwise the same mixes, pre, post, comb and h
    # either way, and hc_mixes alone gives the same mixes.
    n = TWO_PASS_MAX_N + 52
    w = hin.Workload("w%d" % d, 1, n, 4, d, 1.0 / np.sqrt(4 * d), 0.5, 2.0, 1.0)
    t = hin.make_inputs(w, DEV, seed=43)
    full = run_fused(t["R"], t["W"], t["scale"], t["base"])
    for lo, hi in [(0, 1), (7, 40), (52, n), (n - 3, n)]:
        sub = t["R"][:, lo:hi].contiguous()
        part = run_fused(sub, t["W"], t["scale"], t["base"])
        for name, u, v in zip(("h", "pre", "post", "comb", "mixes"), full, part):
            assert torch.equal(u[:, lo:hi], v), (d, lo, hi, name)
        m = hcl.hc_mixes(sub, t["W"])
        torch.cuda.synchronize()
        assert torch.equal(full[4][:, lo:hi], m), (d, lo, hi, "hc_mixes")


@pytest.mark.parametrize("d,n", [(5120, 1), (5120, 64), (5120, 256), (5120, 257), (5120, 2100),
                                 (5120, 4097), (5120, 20011), (5120, 65536),
                                 (256, 3000), (1024, 2049), (2048, 2500), (2560, 2200), (3072, 4133),
                                 (256, 77), (64, 40)])
def test_post_mix_pre_matches_the_two_calls(orc, d, n):
    # hc_post of sublayer l and then the fused call of sublayer l+1 on its
    # output, as one entry point: bitwise the two calls in sequence, out of
    # place and in place (R_out == R), on the two-pass path, on the
    # persistent kernel that forms R' from each round in LDS (every slice
    # width it serves, ragged last rounds, the large workload's size) and at
    # widths of the cooperative kernel.
    w = hin.Workload("pmp%d" % d, 1, n, 4, d, 1.0 / np.sqrt(4 * d), 0.5, 2.0, 1.0)
    t = hin.make_inputs(w, DEV, seed=61)
    nxt = hin.make_inputs(w, DEV, seed=62)          # sublayer l+1's weights, scale and base
    _, _, post, comb, _ = run_fused(t["R"], t["W"], t["scale"], t["base"])
    Rp = hcl.hc_post(t["x"], t["R"], post, comb)
    ref = run_fused(Rp, nxt["W"], nxt["scale"], nxt["base"])
    got = hcl.hc_post_mix_pre(t["x"], t["R"], post, comb, nxt["W"], nxt["scale"], nxt["base"],
                              want_pre=True, want_mixes=True)
    torch.cuda.synchronize()
    assert torch.equal(got[0], Rp)
    for name, u, v in zip(("h", "pre", "post", "comb", "mixes"), got[1:], ref):
        assert torch.equal(u, v), name
    R2 = t["R"].clone()
    got2 = hcl.hc_post_mix_pre(t["x"], R2, post, comb, nxt["W"], nxt["scale"], nxt["base"],
                               want_pre=True, want_mixes=True, out_R=R2)
    torch.cuda.synchronize()
    assert torch.equal(R2, Rp)
    for name, u, v in zip(("h", "pre", "post", "comb", "mixes"), got2[1:], ref):
        assert torch.equal(u, v), name + " (in place)"
    if n <= 64:
        compare_fused(orc, Rp, nxt["W"], nxt["scale"], nxt["base"], tuple(got[1:]), label="post+mix n=%d" % n)


@pytest.mark.parametrize("d,n", [(5120, 1), (5120, 64), (5120, 2048), (5120, 2100), (1024, 77), (256, 300)])
def test_packed_weights_match_unpacked_bitwise(d, n):
    # weights split once by hc_pack_weights give bitwise the results of the
    # call that splits them itself, on the two-pass and the persistent path
    w = hin.Workload("pk%d" % d, 1, n, 4, d, 1.0 / np.sqrt(4 * d), 0.5, 2.0, 1.0)
    t = hin.make_inputs(w, DEV, seed=91)
    packed = hcl.hc_pack_weights(t["W"])
    ref = run_fused(t["R"], t["W"], t["scale"], t["base"])
    got = hcl.hc_fused_mix_pre(t["R"], t["W"], t["scale"], t["base"], want_pre=True, want_mixes=True,
                               packed=packed)
    torch.cuda.synchronize()
    for name, u, v in zip(("h", "pre", "post", "comb", "mixes"), got, ref):
        assert torch.equal(u, v), (d, n, name)


@pytest.mark.parametrize("hc,d,n", [(4, 5120, 64), (4, 5120, 4096), (4, 64, 77), (2, 256, 50), (3, 8, 20_000),
                                    (8, 64, 40)])
def test_graph_capture_replays_bitwise(hc, d, n):
    # the fused call and hc_post captured into one HIP graph, on the
    # two-pass (64 tokens), persistent (4,096) and cooperative (d = 64)
    # paths, and on the plain kernels of other stream counts (all three
    # projection kernels): every replay, with eager calls of the library in
    # between, gives bitwise the eager results
    w = hin.Workload("g%d" % d, 1, n, hc, d, 1.0 / np.sqrt(hc * d), 0.5, 2.0, 1.0)
    M = (2 + hc) * hc
    t = hin.make_inputs(w, DEV, seed=97)
    R, x, W, s, b = t["R"], t["x"], t["W"], t["scale"], t["base"]
    ws = hcl.Workspace()
    outs = dict(h=torch.empty(1, n, d, dtype=torch.bfloat16, device=DEV), pre=torch.empty(1, n, hc, device=DEV),
                post=torch.empty(1, n, hc, device=DEV), comb=torch.empty(1, n, hc, hc, device=DEV),
                mixes=torch.empty(1, n, M, device=DEV))
    Rout = torch.empty_like(R)

    def step():
        hcl.hc_fused_mix_pre(R, W, s, b, want_pre=True, want_mixes=True, workspace=ws, out=outs)
        hcl.hc_post(x, R, outs["post"], outs["comb"], out=Rout)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    ref["Rout"] = Rout.clone()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in list(outs.values()) + [Rout]:
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in list(outs.items()) + [("Rout", Rout)]:
            assert torch.equal(v, ref[k]), (d, n, rep, k)
        hcl.hc_fused_mix_pre(R, W, s, b, workspace=ws)      # eager work between replays
        torch.cuda.synchronize()


def test_workspace_reused_across_shapes():
    # one workspace through calls of different sizes and widths, mixes kept
    # in the workspace: every result equals that of a fresh workspace
    w = hin.WORKLOADS["prefill"]
    t = hin.make_inputs(w, DEV, seed=29)
    w2 = hin.Workload("w2048", 1, 300, 4, 2048, 1.0 / np.sqrt(4 * 2048), 0.5, 2.0, 1.0)
    t2 = hin.make_inputs(w2, DEV, seed=31)
    shared = hcl.Workspace()
    cases = [(t["R"], t), (t["R"][:, :100].contiguous(), t), (t2["R"], t2), (t["R"], t),
             (t["R"][:, :5].contiguous(), t), (t["R"], t)]
    for R, src in cases:
        args = (R, src["W"], src["scale"], src["base"])
        got = hcl.hc_fused_mix_pre(*args, want_pre=True, want_mixes=False, workspace=shared)
        ref = hcl.hc_fused_mix_pre(*args, want_pre=True, want_mixes=False, workspace=hcl.Workspace())
        torch.cuda.synchronize()
        for u, v in zip(got, ref):
            if u is not None:
                assert torch.equal(u, v)


def test_workspace_shared_by_both_projection_kernels():
    # one workspace alternated between the wave-specialised kernel (d = 5120,
    # 2048 with more than 2,048 tokens: it prepares the workspace header
    # itself), the two-pass path (the same widths, fewer tokens: untagged
    # records) and the cooperative kernel (d = 64, 8192: a separate
    # preparation launch), fused and standalone calls mixed: every result
    # equals that of a fresh workspace, so no record of one call is ever
    # taken for another's
    shapes = []
    for i, (d, n) in enumerate([(5120, 2100), (64, 128), (2048, 97), (8192, 159), (5120, 190), (64, 221),
                                (8192, 252), (2048, 2300), (5120, 2200), (5120, 60)]):
        w = hin.Workload("d%d" % d, 1, n, 4, d, 1.0 / np.sqrt(4 * d), 0.5, 2.0, 1.0)
        shapes.append(hin.make_inputs(w, DEV, seed=40 + i))
    shared = hcl.Workspace()
    for i, t in enumerate(shapes):
        args = (t["R"], t["W"], t["scale"], t["base"])
        if i % 3 == 2:
            got = (hcl.hc_mixes(t["R"], t["W"], workspace=shared),)
            ref = (hcl.hc_mixes(t["R"], t["W"], workspace=hcl.Workspace()),)
        else:
            got = hcl.hc_fused_mix_pre(*args, want_pre=True, want_mixes=True, workspace=shared)
            ref = hcl.hc_fused_mix_pre(*args, want_pre=True, want_mixes=True, workspace=hcl.Workspace())
        torch.cuda.synchronize()
        for u, v in zip(got, ref):
            if u is not None:
                assert torch.equal(u, v), "call %d (d=%d)" % (i, t["R"].shape[-1])


def test_zero_and_scaled_tokens(orc):
    w = hin.WORKLOADS["decode"]
    t = hin.make_inputs(w, DEV, seed=19)
    R = t["R"].clone()
    R[3] = 0                                   # an all-zero token: mixes exactly 0
    R[5] = R[4] * 2.0 ** 40                    # power-of-two scaled copies
    R[6] = R[4] * 2.0 ** -20                   # (mean square still far above norm_eps)
    h, pre, post, comb, mixes = run_fused(R, t["W"], t["scale"], t["base"])
    assert torch.equal(mixes[3, 0], torch.zeros_like(mixes[3, 0]))
    assert bool(torch.isfinite(mixes).all())
    check_mixes(_np(mixes[5, 0]), _np(mixes[4, 0]).astype(np.float64), tol=1e-6)
    check_mixes(_np(mixes[6, 0]), _np(mixes[4, 0]).astype(np.float64), tol=1e-6)
    # moderate power-of-two scales leave the mixes unchanged bit for bit, so
    # h and R' scale exactly
    assert torch.equal(mixes[5], mixes[4])
    assert torch.equal(h[5].float(), h[4].float() * 2.0 ** 40)
    compare_fused(orc, R, t["W"], t["scale"], t["base"], (h, pre, post, comb, mixes), x=t["x"], label="scaled")


@pytest.mark.parametrize("d", [64, 1024, 5120])
def test_huge_tokens_sum_of_squares_overflow(orc, d):
    """Streams whose squares overflow fp32 (a chained stack without a norm
    grows by about e per sublayer): at 2^56 the plain fp32 sum of squares is
    still finite, from about 2^58 on it overflows and the scaled sum takes
    over; up to 2^124 the bf16 values themselves stay finite."""
    w = hin.WORKLOADS["decode"]
    t = hin.make_inputs(w, DEV, seed=29)
    R = t["R"][..., :d].contiguous().clone()
    W, s, b = hin.make_params(w, DEV, seed=29)
    W = W.view(-1, 4, w.d)[:, :, :d].contiguous().view(-1, 4 * d)
    exps = [56, 60, 64, 80, 100, 120, 124]
    for i, e in enumerate(exps):
        R[8 + i] = R[i] * 2.0 ** e
    h, pre, post, comb, mixes = run_fused(R, W, s, b)
    assert bool(torch.isfinite(mixes).all())
    for i, e in enumerate(exps):
        check_mixes(_np(mixes[8 + i, 0]), _np(mixes[i, 0]).astype(np.float64), tol=1e-6)
    x = t["x"][..., :d].contiguous()
    compare_fused(orc, R, W, s, b, (h, pre, post, comb, mixes), x=x, label="huge d=%d" % d)
    # the standalone projection agrees bit for bit with the fused call
    assert torch.equal(hcl.hc_mixes(R, W), mixes)


def test_diag_scale_bitwise(orc):
    w = hin.WORKLOADS["prefill"]
    h = hin.make_inputs(w, DEV, seed=23, n_tokens=300)["x"]
    D = hin.make_diag(hin.WORKLOADS["chained"], 0, DEV)
    x = hcl.hc_diag_scale(h, D)
    torch.cuda.synchronize()
    check_bf16_exact(hin.bits(x).reshape(300, -1),
                     orc.diag_scale(hin.bits(h).reshape(300, -1), hin.bits(D)), "diag_scale")


def test_errors_are_raised_on_gpu():
    w = hin.WORKLOADS["tiny"]
    t = hin.make_inputs(w, DEV)
    import ctypes
    lib = hcl.load()
    n, d = w.n, w.d
    h = torch.empty(n, d, dtype=torch.bfloat16, device=DEV)
    post = torch.empty(n, 4, device=DEV)
    comb = torch.empty(n, 4, 4, device=DEV)
    ws = torch.empty(4096, dtype=torch.uint8, device=DEV)
    off = (-ws.data_ptr()) % 256
    P = lambda t_: ctypes.c_void_p(t_.data_ptr())
    st = lib.hc_fused_mix_pre(P(t["R"]), P(t["W"]), P(t["scale"]), P(t["base"]), P(h), None, P(post), P(comb),
                              None, ctypes.c_void_p(ws.data_ptr() + off), 256, n, 4, d, 20, 1e-6, 1e-20, None)
    assert st == -5          # workspace too small: refused before any launch
    with pytest.raises(hcl.HCError):
        hcl.hc_split_sinkhorn(torch.zeros(4, 24, device=DEV), t["scale"], t["base"], sinkhorn_iters=0)
    with pytest.raises(ValueError):
        hcl.hc_pre(t["R"].cpu(), torch.zeros(1, 16, 4))


# ------------------------------------------------- stream counts other than 4
# The split + Sinkhorn listing and the mix formula are written for any hc;
# hc = 1..8 other than 4 run the plain kernels of hc_general.hip.

def _hc_workload(hc, d):
    return dataclasses.replace(hin.WORKLOADS["prefill"], hc=hc, d=d)


@pytest.mark.parametrize("hc,d,n", [(1, 64, 37), (2, 256, 100), (3, 5120, 33), (5, 128, 65), (6, 512, 40),
                                    (7, 64, 17), (8, 5120, 70)])
def test_other_stream_counts(orc, hc, d, n):
    w = _hc_workload(hc, d)
    t = hin.make_inputs(w, DEV, seed=11, n_tokens=n)
    R = t["R"]
    R[0, 0].zero_()                                   # an all-zero token: mixes exactly 0
    if n > 1:
        R[0, 1].mul_(2.0 ** 100)                      # squares far beyond the float range
    outs = run_fused(R, t["W"], t["scale"], t["base"])
    assert bool((outs[4][0, 0] == 0).all())
    compare_fused(orc, R, t["W"], t["scale"], t["base"], outs, x=t["x"], label="hc=%d d=%d" % (hc, d))
    # the standalone entry points give the fused call's results bit for bit
    h, pre, post, comb, mixes = outs
    m2 = hcl.hc_mixes(R, t["W"])
    p2, q2, c2 = hcl.hc_split_sinkhorn(m2, t["scale"], t["base"], hc_mult=hc)
    h2 = hcl.hc_pre(R, p2)
    torch.cuda.synchronize()
    for a, b in ((m2, mixes), (p2, pre), (q2, post), (c2, comb)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(h2.view(torch.int16), h.view(torch.int16))


@pytest.mark.parametrize("hc", [2, 8])
def test_post_mix_pre_other_stream_counts(hc):
    w = _hc_workload(hc, 256)
    t = hin.make_inputs(w, DEV, seed=12, n_tokens=50)
    _, _, post, comb, _ = run_fused(t["R"], t["W"], t["scale"], t["base"])
    W2, s2, b2 = hin.make_params(w, DEV, seed=13)
    R1 = hcl.hc_post(t["x"], t["R"], post, comb)
    a = hcl.hc_fused_mix_pre(R1, W2, s2, b2, want_mixes=True)
    Rc = t["R"].clone()
    Ro, *b = hcl.hc_post_mix_pre(t["x"], Rc, post, comb, W2, s2, b2, want_mixes=True, out_R=Rc)
    torch.cuda.synchronize()
    assert Ro.data_ptr() == Rc.data_ptr()
    assert torch.equal(Ro.view(torch.int16), R1.view(torch.int16))
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


@pytest.mark.parametrize("hc,d,n", [(2, 64, 140_001), (3, 8, 140_001), (6, 8, 140_001), (3, 72, 9_001),
                                    (2, 5120, 65_536), (3, 5120, 65_536), (8, 5120, 65_536)])
def test_other_stream_count_many_tiles_sampled(orc, hc, d, n):
    # the matrix-core projection with one workgroup per 256-token tile taking
    # every segment of the reduction axis (at least as many tiles as compute
    # units), sampled against the oracle: reduction axes shorter than one
    # staged chunk (d = 8), not a multiple of it (hc = 3, d = 72), and the
    # large workload's 65,536 tokens at d = 5120
    w = _hc_workload(hc, d)
    t = hin.make_inputs(w, DEV, seed=14, n_tokens=n)
    outs = run_fused(t["R"], t["W"], t["scale"], t["base"])
    idx = np.concatenate([hin.sample_tokens(n, 200), [n - 1]])
    compare_fused(orc, t["R"], t["W"], t["scale"], t["base"], outs, idx=idx, x=t["x"], label="hc=%d n=140001" % hc)


@pytest.mark.parametrize("hc,d,n,span", [(2, 256, 101, 37), (5, 64, 20_001, 37), (3, 8, 50_001, 1_000),
                                         (8, 64, 101, 37), (6, 8, 20_001, 300), (8, 8, 17_001, 40),
                                         (2, 5120, 70_000, 37), (3, 1024, 70_000, 5_000), (8, 512, 70_000, 300),
                                         (7, 256, 66_000, 20_000)])
def test_other_stream_counts_batch_invariant_and_deterministic(hc, d, n, span):
    # a token's results do not depend on the other tokens of its call, and
    # repeated calls agree bit for bit, whichever way the projection runs:
    # long calls (70,000 tokens: at least a tile of 256 per compute unit) have
    # one workgroup per tile add every segment of the reduction axis, shorter
    # ones one workgroup per segment with the partial sums added afterwards,
    # and the tile size (32 .. 256 tokens) follows the call's size.
    w = _hc_workload(hc, d)
    t = hin.make_inputs(w, DEV, seed=15, n_tokens=n)
    lo = n // 3 + 1
    hi = lo + span
    full = run_fused(t["R"], t["W"], t["scale"], t["base"])
    again = run_fused(t["R"], t["W"], t["scale"], t["base"])
    part = run_fused(t["R"][:, lo:hi].contiguous(), t["W"], t["scale"], t["base"])
    for a, b, c in zip(full, again, part):
        iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(iv), b.view(iv))
        assert torch.equal(a[:, lo:hi].contiguous().view(iv), c.view(iv))


def test_other_stream_count_call_invalidates_four_stream_header():
    # a workspace shared across stream counts: a call at hc != 4 zeroes the
    # first 256 bytes (a four-stream call's header), even when it takes one
    # workgroup per tile (no partial sums written) with the mixes kept by the
    # caller, so a later four-stream call clears its record area instead of
    # trusting stale contents, and gives the fresh-workspace bits
    ws = hcl.Workspace()
    w4 = _hc_workload(4, 256)
    t4 = hin.make_inputs(w4, DEV, seed=21, n_tokens=3000)
    first = hcl.hc_fused_mix_pre(t4["R"], t4["W"], t4["scale"], t4["base"], workspace=ws, want_mixes=True)
    w3 = _hc_workload(3, 64)
    t3 = hin.make_inputs(w3, DEV, seed=22, n_tokens=70000)
    hcl.hc_fused_mix_pre(t3["R"], t3["W"], t3["scale"], t3["base"], workspace=ws, want_pre=False, want_mixes=True)
    torch.cuda.synchronize()
    head = ws._buf[ws._off:ws._off + 256]
    assert int(head.count_nonzero()) == 0, "the four-stream header survived a three-stream call"
    again = hcl.hc_fused_mix_pre(t4["R"], t4["W"], t4["scale"], t4["base"], workspace=ws, want_mixes=True)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        iv = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(a.view(iv), b.view(iv))


@pytest.mark.parametrize("d", [5120, 2048, 64])
def test_post_short_and_long_calls_agree_bitwise(d):
    # hc_post takes half-chunk items (k_post4) for calls with fewer 16-byte
    # items than one workgroup per CU and full chunks (k_post) beyond: a
    # token's R' is the same bits whichever kernel its call runs, in place
    # or not
    g = torch.Generator(device="cpu").manual_seed(61)
    n = 2 * 256 * torch.cuda.get_device_properties(0).multi_processor_count * 8 // d + 40
    R = torch.randn(n, 4, d, generator=g).to(torch.bfloat16).to(DEV)
    x = torch.randn(n, d, generator=g).to(torch.bfloat16).to(DEV)
    post = (2 * torch.rand(n, 4, generator=g)).to(DEV)
    comb = torch.rand(n, 4, 4, generator=g).to(DEV)
    full = hcl.hc_post(x, R, post, comb)
    for lo, hi in [(0, 1), (3, 67), (0, n // 3), (n // 3, n)]:
        part = hcl.hc_post(x[lo:hi].contiguous(), R[lo:hi].contiguous(), post[lo:hi].contiguous(),
                           comb[lo:hi].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(full[lo:hi], part), (d, lo, hi)
    Rin = R[:5].clone()
    hcl.hc_post(x[:5].contiguous(), Rin, post[:5].contiguous(), comb[:5].contiguous(), out=Rin)
    torch.cuda.synchronize()
    assert torch.equal(full[:5], Rin), (d, "in place")
