"""GPU parity of the pre-sublayer RMSNorm: hc_rmsnorm and hc_pre_norm (hc_pre
and the norm in one pass over R) against the fp64 oracle, through the
C-ABI.  h must equal the oracle's hc_pre bit for bit; y is graded by
tests/hc_check.py check_norm (1 bf16 ulp, and bit for bit but for the rare
output that the order of the double sum of squares moves).

The norm's formula is a reading of the "Mix projection" page (the page
builds RMSNorm(dim, norm_eps) and prints no formula): the mix formula's
root-mean-square normalisation over the d features of hc_pre's bf16 output,
times an fp32 per-feature weight.
"""
import numpy as np
import pytest
import torch

import hyper_connection_residual_02_amd as hcl
import oracle
from hyper_connection_residual_02_amd import inputs as hin
from hc_check import check_bf16_exact, check_norm

pytestmark = pytest.mark.gpu
DEV = "cuda"
NEPS = float(np.float32(1e-20))    # the kernels take norm_eps as fp32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hcl.load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _pre(n, hc, seed):
    # pre as the split produces it: sigmoid gates plus hc_eps, in (0, 1]
    return hin.uniform((n, hc), 0.01, 1.0, DEV, seed, 5)


@pytest.mark.parametrize("d,n", [(8, 5), (64, 9), (504, 3), (512, 4), (2048, 7), (2056, 5), (4096, 6),
                                 (5120, 37), (5120, 1), (8200, 5), (16384, 3), (32768, 3)])
def test_rmsnorm_matches_oracle(d, n):
    h = hin.randn((n, d), 1.0, DEV, 11, 1, torch.bfloat16)
    g = hin.make_gamma(d, DEV)
    y = hcl.hc_rmsnorm(h, g, NEPS)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(hin.bits(h), g.cpu().numpy(), NEPS)
    print("d=%d n=%d: %d outputs 1 ulp off" % (d, n, check_norm(hin.bits(y), ref, "y")))


@pytest.mark.parametrize("hc,d,n", [(4, 5120, 37), (4, 5120, 4097), (1, 5120, 9), (2, 5120, 9), (3, 5120, 9),
                                    (5, 5120, 9), (6, 5120, 9), (7, 5120, 9), (8, 5120, 9), (4, 64, 13),
                                    (4, 2056, 6), (4, 8192, 5), (3, 1000, 7)])
def test_pre_norm_matches_oracle(hc, d, n):
    R = hin.randn((n, hc, d), 1.0, DEV, 12, 1, torch.bfloat16)
    pre = _pre(n, hc, 12)
    g = hin.make_gamma(d, DEV)
    y, h = hcl.hc_pre_norm(R, pre, g, NEPS, want_h=True)
    h_sep = hcl.hc_pre(R, pre)
    y_only = hcl.hc_pre_norm(R, pre, g, NEPS)
    torch.cuda.synchronize()
    hb = oracle.pre(hin.bits(R), pre.cpu().numpy().astype(np.float64))
    check_bf16_exact(hin.bits(h), hb, "h")
    check_bf16_exact(hin.bits(h_sep), hb, "h (hc_pre)")
    ref = oracle.rmsnorm(hb, g.cpu().numpy(), NEPS)
    off = check_norm(hin.bits(y), ref, "y")
    check_bf16_exact(hin.bits(y_only), hin.bits(y), "y without h")
    print("hc=%d d=%d n=%d: %d outputs 1 ulp off" % (hc, d, n, off))


def test_pre_norm_full_size_sampled():
    # the large prefill workload: 65,536 tokens of 4 x 5120 streams, checked
    # on sampled tokens (every sampled token's h bit for bit, y to check_norm)
    n, hc, d = 65536, 4, 5120
    R = hin.randn((n, hc, d), 1.0, DEV, 13, 1, torch.bfloat16)
    pre = _pre(n, hc, 13)
    g = hin.make_gamma(d, DEV)
    y, h = hcl.hc_pre_norm(R, pre, g, NEPS, want_h=True)
    torch.cuda.synchronize()
    idx = hin.sample_tokens(n, 200, seed=3)
    ti = torch.from_numpy(idx).to(DEV)
    Rs = hin.bits(R.index_select(0, ti))
    hb = oracle.pre(Rs, pre.index_select(0, ti).cpu().numpy().astype(np.float64))
    check_bf16_exact(hin.bits(h.index_select(0, ti)), hb, "h")
    check_norm(hin.bits(y.index_select(0, ti)), oracle.rmsnorm(hb, g.cpu().numpy(), NEPS), "y")


def test_norm_special_tokens():
    d = 5120
    rows = [np.zeros(d), np.full(d, 2.0 ** 120), np.full(d, -(2.0 ** -100)), np.full(d, 3.0)]
    alt = np.ones(d)
    alt[::2] = -1e-30
    rows.append(alt)
    rows.append(np.where(np.arange(d) == 77, 1e30, 1e-30))      # one dominant feature
    hb = hin.bits(torch.tensor(np.stack(rows), dtype=torch.float32).to(torch.bfloat16))
    h = hin.from_bits(hb, DEV)
    g = hin.make_gamma(d, DEV)
    gz = g.clone()
    gz[::3] = 0.0
    gz[1::7] *= -1.0
    for gamma in (g, gz):
        gn = gamma.cpu().numpy()
        for eps in (NEPS, 0.0, 1.0):
            y = hcl.hc_rmsnorm(h, gamma, eps)
            torch.cuda.synchronize()
            ref = oracle.rmsnorm(hb, gn, eps)
            check_norm(hin.bits(y), ref, "y eps=%g" % eps)
            if eps > 0:
                assert ((hin.bits(y[0]) & 0x7FFF) == 0).all()       # zero token -> zeros
            else:
                assert ((hin.bits(y[0]) & 0x7FFF) > 0x7F80).all()   # 0 / 0, as the definition gives


def test_norm_batch_invariant():
    # a token's y does not depend on how many tokens share the call
    d = 5120
    h = hin.randn((3000, d), 1.0, DEV, 14, 1, torch.bfloat16)
    g = hin.make_gamma(d, DEV)
    full = hcl.hc_rmsnorm(h, g, NEPS)
    for m in (1, 3, 5, 2999):
        part = hcl.hc_rmsnorm(h[:m].contiguous(), g, NEPS)
        torch.cuda.synchronize()
        check_bf16_exact(hin.bits(part), hin.bits(full[:m]), "y of %d tokens" % m)


# ------------------------------------------------- hc_fused_mix_pre_norm
# The fused kernels (every path: two-pass, wave-specialised, other widths,
# other stream counts), then the norm kernel on h, or in place on y when h
# is not kept.  The coefficients and h are bitwise hc_fused_mix_pre's, and y
# is graded against the oracle's norm of that h.

import dataclasses


def _wl(hc, d):
    return dataclasses.replace(hin.WORKLOADS["prefill"], hc=hc, d=d)


def _fused_norm_case(hc, d, n, seed, want_h, sample=None):
    w = _wl(hc, d)
    t = hin.make_inputs(w, DEV, seed=seed, n_tokens=n)
    g = hin.make_gamma(d, DEV, seed=seed)
    y, h, pre, post, comb, mixes = hcl.hc_fused_mix_pre_norm(t["R"], t["W"], t["scale"], t["base"], g,
                                                             norm_eps=NEPS, want_h=want_h, want_mixes=True)
    ref = hcl.hc_fused_mix_pre(t["R"], t["W"], t["scale"], t["base"], norm_eps=NEPS, want_mixes=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("pre", "post", "comb", "mixes"), (pre, post, comb, mixes), ref[1:]):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    if want_h:
        assert torch.equal(h.view(torch.int16), ref[0].view(torch.int16)), "h"
    idx = np.arange(n) if sample is None else hin.sample_tokens(n, sample, seed=seed)
    ti = torch.from_numpy(idx).to(DEV)
    hb = hin.bits(ref[0].reshape(n, d).index_select(0, ti))
    off = check_norm(hin.bits(y.reshape(n, d).index_select(0, ti)), oracle.rmsnorm(hb, g.cpu().numpy(), NEPS), "y")
    return t, g, y, off


@pytest.mark.parametrize("hc,d,n,want_h", [
    (4, 5120, 2049, False), (4, 5120, 4097, True), (4, 5120, 20011, False),   # persistent kernel, ragged tails
    (4, 2560, 3000, True), (4, 1024, 2500, False), (4, 256, 2200, True),      # other wave-specialised widths
    (4, 5120, 64, False), (4, 5120, 2048, True),                              # two-pass path + norm kernel
    (4, 64, 300, True), (4, 6144, 2100, False),                               # other widths (k_coop)
    (2, 5120, 3000, False), (3, 1000, 37, True), (8, 512, 2100, False)])      # other stream counts
def test_fused_norm_matches_oracle(hc, d, n, want_h):
    _fused_norm_case(hc, d, n, 21, want_h)


def test_fused_norm_full_size_sampled():
    # the large prefill workload (65,536 tokens x 4 x 5120), in the launch
    # configuration the benchmark times, on sampled tokens
    _fused_norm_case(4, 5120, 65536, 22, False, sample=300)


def test_fused_norm_agrees_with_pre_norm_and_is_deterministic():
    # the fused call's norm and the one-pass hc_pre_norm on the same pre
    # (one ulp at most: their sums of squares run in different orders);
    # repeated calls agree bit for bit, and a token's y does not depend on
    # the other tokens of its call
    n, d = 20011, 5120
    t, g, y, _ = _fused_norm_case(4, d, n, 23, False)
    y2 = hcl.hc_fused_mix_pre_norm(t["R"], t["W"], t["scale"], t["base"], g, norm_eps=NEPS)[0]
    lo, hi = 5000, 5000 + 3001
    y3 = hcl.hc_fused_mix_pre_norm(t["R"][:, lo:hi].contiguous(), t["W"], t["scale"], t["base"], g,
                                   norm_eps=NEPS)[0]
    pre = hcl.hc_fused_mix_pre(t["R"], t["W"], t["scale"], t["base"], norm_eps=NEPS)[1]
    yp = hcl.hc_pre_norm(t["R"].reshape(n, 4, d), pre.reshape(n, 4), g, NEPS)
    torch.cuda.synchronize()
    check_bf16_exact(hin.bits(y2), hin.bits(y), "y, second call")
    check_bf16_exact(hin.bits(y3), hin.bits(y[:, lo:hi].contiguous()), "y of a slice")
    check_norm(hin.bits(yp), hin.bits(y).reshape(n, d), "y vs hc_pre_norm")


def test_fused_norm_graph_replay():
    # captured once, replayed three times with eager work between replays:
    # every replay equals the eager call
    n, d = 4097, 5120
    w = _wl(4, d)
    t = hin.make_inputs(w, DEV, seed=24, n_tokens=n)
    g = hin.make_gamma(d, DEV, seed=24)
    ws = hcl.Workspace(DEV)
    eager = hcl.hc_fused_mix_pre_norm(t["R"], t["W"], t["scale"], t["base"], g, norm_eps=NEPS, workspace=ws)[0]
    out = {"y": torch.empty_like(eager), "post": torch.empty(1, n, 4, device=DEV),
           "comb": torch.empty(1, n, 4, 4, device=DEV), "pre": torch.empty(1, n, 4, device=DEV)}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            hcl.hc_fused_mix_pre_norm(t["R"], t["W"], t["scale"], t["base"], g, norm_eps=NEPS, workspace=ws,
                                      out=out)
    torch.cuda.current_stream().wait_stream(s)
    for k in range(3):
        out["y"].zero_()
        graph.replay()
        hcl.hc_rmsnorm(eager.reshape(n, d), g, NEPS)      # eager work between replays
        torch.cuda.synchronize()
        check_bf16_exact(hin.bits(out["y"]), hin.bits(eager), "replay %d" % k)
