"""Pins of the oracle's backward pass against things other than itself.

The pages give the forward only; the gradient of a scalar loss through it
is fixed by the mathematics.  The oracle's backward (chain rule over the
forward's steps in reverse order) is pinned here by:

* central finite differences of the forward in fp64 -- for the split and
  Sinkhorn through the (separately pinned) forward oracle, for the whole
  sublayer through a numpy projection feeding it -- with a fourth-order
  stencil, so that a dropped term, a wrong sign, a transposed operand or a
  wrong index shows as an error many orders above the tolerance;
* a 50-digit mpmath finite difference of the listing's steps, written out
  on their own in mpmath (independent of the fp64 oracle), for one token;
* identities the chain rule fixes: z = s m + b gives s * gscale = sum m gm
  and gbase = gm summed over tokens, group by group (pre, post, comb);
* invariances: comb does not change when a constant is added to a row of
  logits, so each row of the comb logits' gradients sums to zero; the
  mixes do not change when a token's stream is scaled (norm_eps = 0), so
  the projection's share of dL/dR is orthogonal to the stream;
* the gradient of the weights is additive over tokens; at W = 0 the
  projection passes no gradient to R.
"""
import mpmath
import numpy as np
import pytest
import torch

import oracle

mpmath.mp.dps = 50


def bf16_bits(a):
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return oracle.bf16_to_f64(bits)


def draw(n, hc, d, seed, w_std=0.3, s_lo=0.5, s_hi=2.0, b_std=1.0):
    rng = np.random.default_rng(seed)
    M = (2 + hc) * hc
    R = bf16_bits(rng.standard_normal((n, hc, d)))
    x = bf16_bits(rng.standard_normal((n, d)))
    gRo = bf16_bits(rng.standard_normal((n, hc, d)))
    gh = bf16_bits(rng.standard_normal((n, d)))
    W = (rng.standard_normal((M, hc * d)) * w_std).astype(np.float32)
    s = rng.uniform(s_lo, s_hi, 3).astype(np.float32)
    b = (rng.standard_normal(M) * b_std).astype(np.float32)
    return R, x, gRo, gh, W, s, b


def fd4(f, v, h):
    """Fourth-order central difference of f along the unit direction at v."""
    return (-f(v + 2 * h) + 8 * f(v + h) - 8 * f(v - h) + f(v - 2 * h)) / (12 * h)


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


# ------------------------------------------------------------ split + Sinkhorn

def split_loss(m, s, b, gp, gq, gc, hc, iters, eps):
    p, q, c = oracle.split_sinkhorn(m[None, :], s, b, hc, iters, eps)
    return float(np.sum(gp * p[0]) + np.sum(gq * q[0]) + np.sum(gc * c[0]))


@pytest.mark.parametrize("hc,iters,eps,s2", [(4, 20, 1e-6, 2.0), (4, 1, 1e-6, 1.0), (4, 2, 0.0, 1.0),
                                             (4, 20, 1e-3, 20.0), (2, 7, 1e-6, 5.0), (3, 20, 1e-6, 1.0),
                                             (8, 20, 1e-6, 1.0), (1, 20, 1e-6, 1.0)])
def test_split_backward_matches_finite_differences(hc, iters, eps, s2):
    rng = np.random.default_rng(100 + hc * 10 + iters)
    M = (2 + hc) * hc
    m = rng.standard_normal(M)
    s = np.array([rng.uniform(0.5, 2), rng.uniform(0.5, 2), s2], np.float32)
    b = rng.standard_normal(M).astype(np.float32)
    gp, gq, gc = rng.standard_normal(hc), rng.standard_normal(hc), rng.standard_normal((hc, hc))
    gm, gs, gb, _, _ = oracle.split_sinkhorn_backward(m[None], s, b, gp[None], gq[None], gc[None], hc, iters, eps)
    num = np.empty(M)
    for i in range(M):
        e = np.zeros(M)
        e[i] = 1.0
        num[i] = fd4(lambda t: split_loss(m + t * e, s, b, gp, gq, gc, hc, iters, eps), 0.0, 1e-3)
    assert rel_err(gm[0], num) < 1e-8, rel_err(gm[0], num)


def _sink_mp(m, s, b, hc, iters, eps):
    """The listing's steps in mpmath: gates, row softmax + eps, a column
    normalisation, then (iters - 1) row and column normalisations."""
    pre = [1 / (1 + mpmath.exp(-(s[0] * m[j] + b[j]))) + eps for j in range(hc)]
    post = [2 / (1 + mpmath.exp(-(s[1] * m[hc + j] + b[hc + j]))) for j in range(hc)]
    C = [[s[2] * m[2 * hc + j * hc + k] + b[2 * hc + j * hc + k] for k in range(hc)] for j in range(hc)]
    for j in range(hc):
        ex = [mpmath.exp(v) for v in C[j]]
        z = mpmath.fsum(ex)
        C[j] = [v / z + eps for v in ex]

    def col():
        for k in range(hc):
            z = mpmath.fsum(C[j][k] for j in range(hc)) + eps
            for j in range(hc):
                C[j][k] = C[j][k] / z

    def row():
        for j in range(hc):
            z = mpmath.fsum(C[j]) + eps
            C[j] = [v / z for v in C[j]]
    col()
    for _ in range(iters - 1):
        row()
        col()
    return pre, post, C


@pytest.mark.parametrize("hc,s2", [(4, 20.0), (2, 3.0)])
def test_split_backward_matches_mpmath_finite_differences(hc, s2):
    rng = np.random.default_rng(7 + hc)
    M = (2 + hc) * hc
    iters, eps = 20, 1e-6
    m = rng.standard_normal(M)
    s = np.array([1.3, 0.7, s2], np.float32)
    b = rng.standard_normal(M).astype(np.float32)
    gp, gq, gc = rng.standard_normal(hc), rng.standard_normal(hc), rng.standard_normal((hc, hc))
    gm = oracle.split_sinkhorn_backward(m[None], s, b, gp[None], gq[None], gc[None], hc, iters, eps)[0][0]
    S = [mpmath.mpf(float(v)) for v in s]
    B = [mpmath.mpf(float(v)) for v in b]
    E = mpmath.mpf(eps)

    def loss(mm):
        pre, post, C = _sink_mp(mm, S, B, hc, iters, E)
        return (mpmath.fsum(mpmath.mpf(gp[j]) * pre[j] for j in range(hc)) +
                mpmath.fsum(mpmath.mpf(gq[j]) * post[j] for j in range(hc)) +
                mpmath.fsum(mpmath.mpf(gc[j, k]) * C[j][k] for j in range(hc) for k in range(hc)))
    h = mpmath.mpf("1e-20")
    base = [mpmath.mpf(float(v)) for v in m]
    num = []
    for i in range(M):
        up = list(base); up[i] += h
        dn = list(base); dn[i] -= h
        num.append(float((loss(up) - loss(dn)) / (2 * h)))
    assert rel_err(gm, num) < 1e-11, rel_err(gm, num)


@pytest.mark.parametrize("hc", [1, 2, 4, 5])
def test_split_backward_chain_rule_identities_and_row_shift(hc):
    rng = np.random.default_rng(31 + hc)
    n, M = 5, (2 + hc) * hc
    m = rng.standard_normal((n, M))
    s = rng.uniform(0.5, 2.0, 3).astype(np.float32)
    b = rng.standard_normal(M).astype(np.float32)
    gp, gq, gc = rng.standard_normal((n, hc)), rng.standard_normal((n, hc)), rng.standard_normal((n, hc, hc))
    gm, gs, gb, gs_t, gb_t = oracle.split_sinkhorn_backward(m, s, b, gp, gq, gc, hc, 20, 1e-6)
    groups = [slice(0, hc), slice(hc, 2 * hc), slice(2 * hc, M)]
    for gi, sl in enumerate(groups):
        # z = s m + b: s * dL/ds = sum m dL/dm, and dL/db = dL/dz = dL/dm / s
        assert np.isclose(float(s[gi]) * gs[gi], np.sum(m[:, sl] * gm[:, sl]), rtol=1e-12, atol=1e-14)
        assert np.allclose(gb[sl] * float(s[gi]), gm[:, sl].sum(0), rtol=1e-12, atol=1e-14)
    assert np.allclose(gs, gs_t.sum(0), rtol=1e-14) and np.allclose(gb, gb_t.sum(0), rtol=1e-14)
    # adding a constant to a row of logits leaves comb unchanged
    rows = gm[:, 2 * hc:].reshape(n, hc, hc).sum(-1)
    assert np.max(np.abs(rows)) <= 1e-12 * max(1.0, np.max(np.abs(gm)))


# ------------------------------------------------------------ whole sublayer

def forward_real(R, x, W, s, b, hc, iters, eps, ne):
    """The forward on real-valued inputs (no bf16 rounding of h and R'):
    numpy projection, the oracle's split + Sinkhorn, hc_pre and hc_post."""
    n = R.shape[0]
    K = R.shape[1] * R.shape[2]
    X = R.reshape(n, K)
    r = 1.0 / np.sqrt((X * X).sum(1) / K + ne)
    m = (X @ W.T) * r[:, None]
    p, q, c = oracle.split_sinkhorn(m, s, b, hc, iters, eps)
    h = np.einsum("tk,tkc->tc", p, R)
    Rp = q[:, :, None] * x[:, None, :] + np.einsum("tjk,tjc->tkc", c, R)
    return h, Rp


@pytest.mark.parametrize("n,hc,d,ne", [(2, 4, 4, 1e-20), (3, 2, 8, 1e-20), (1, 3, 4, 0.5)])
def test_full_backward_matches_finite_differences(n, hc, d, ne):
    R, x, gRo, gh, W, s, b = draw(n, hc, d, seed=50 + hc + d)
    iters, eps = 20, 1e-6
    g = oracle.backward(R, x, W, s, b, gRo, gh, iters, eps, ne)
    Rf, xf, Wf = f64(R), f64(x), W.astype(np.float64)
    gRf, ghf = f64(gRo), f64(gh)

    def loss(Rv, xv, Wv):
        h, Rp = forward_real(Rv, xv, Wv, s, b, hc, iters, eps, ne)
        return float(np.sum(ghf * h) + np.sum(gRf * Rp))

    for name, base, ana, step in (("R", Rf, g["gR"], 1e-3), ("x", xf, g["gx"], 1e-3), ("W", Wf, g["gW"], 1e-3)):
        num = np.empty(base.size)
        flat = base.reshape(-1)
        for i in range(flat.size):
            def f(tv, i=i):
                v = flat.copy()
                v[i] += tv
                args = {"R": Rf, "x": xf, "W": Wf}
                args[name] = v.reshape(base.shape)
                return loss(args["R"], args["x"], args["W"])
            num[i] = fd4(f, 0.0, step)
        err = rel_err(ana.reshape(-1), num)
        assert err < 1e-8, (name, err)


def test_projection_share_is_orthogonal_to_the_stream():
    # m(a X) = m(X) when norm_eps = 0, so d/da L(a X) = <X, dL/dX (projection)> = 0
    n, hc, d = 4, 4, 16
    R, x, gRo, gh, W, s, b = draw(n, hc, d, seed=77)
    gm = np.random.default_rng(78).standard_normal((n, (2 + hc) * hc))
    gR, _ = oracle.mixes_backward(R, W, gm, 0.0)
    X = f64(R)
    for t in range(n):
        dot = float(np.sum(X[t] * gR[t]))
        assert abs(dot) <= 1e-12 * np.linalg.norm(X[t]) * np.linalg.norm(gR[t])


def test_weight_gradient_is_additive_over_tokens_and_zero_weights_pass_nothing_to_R():
    n, hc, d = 3, 2, 8
    R, x, gRo, gh, W, s, b = draw(n, hc, d, seed=81)
    gm = np.random.default_rng(82).standard_normal((n, (2 + hc) * hc))
    _, gW = oracle.mixes_backward(R, W, gm)
    parts = sum(oracle.mixes_backward(R[t:t + 1], W, gm[t:t + 1])[1] for t in range(n))
    assert np.allclose(gW, parts, rtol=1e-13, atol=1e-15)
    gR0, _ = oracle.mixes_backward(R, np.zeros_like(W), gm)
    assert np.all(gR0 == 0.0)


def test_post_and_pre_backward_special_cases():
    n, hc, d = 2, 4, 8
    R, x, gRo, gh, W, s, b = draw(n, hc, d, seed=90)
    # comb = I, post = 0: hc_post is the identity on R, so dL/dR = dL/dR'
    I = np.broadcast_to(np.eye(hc), (n, hc, hc)).copy()
    gx, gq, gc, gR = oracle.post_backward(x, R, np.zeros((n, hc)), I, gRo)
    assert np.array_equal(gR, f64(gRo)) and np.all(gx == 0.0)
    # one-hot pre: h = R_k, so dL/dR_k = dL/dh and the other streams get nothing
    onehot = np.zeros((n, hc))
    onehot[:, 2] = 1.0
    gp, gRp = oracle.pre_backward(R, onehot, gh)
    assert np.array_equal(gRp[:, 2], f64(gh)) and np.all(gRp[:, [0, 1, 3]] == 0.0)
