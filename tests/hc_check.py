"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (from the workload statement; derivations in the design doc):
* mixes: normwise per token, |dm_j| <= 1e-5 * max_j' |m_ref,j'|;
* pre, post, comb: <= 1e-5 absolute;
* bf16 outputs: 1 bf16 ulp, where an output whose exact value lies far below
  the sum of the magnitudes of its terms (cancellation) may instead differ by
  ulp(y_ref) + 1e-5 * sum|terms| -- the coefficient tolerance carried through
  the sum.  When the oracle is fed the GPU's own fp32 coefficients the bf16
  outputs must match bit for bit (both sides round the exact sum once).
"""
import numpy as np

MIX_TOL = 1e-5
COEF_TOL = 1e-5


def bf16_f64(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ordered(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_dist(a, b):
    return np.abs(ordered(a) - ordered(b))


def bf16_ulp(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_mixes(got, ref, tol=MIX_TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    err = np.abs(got - ref) / np.maximum(scale, 1e-300)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, "mixes normwise error %.3g > %.1g" % (worst, tol)
    return worst


def check_abs(got, ref, name, tol=COEF_TOL):
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    worst = float(d.max()) if d.size else 0.0
    assert worst <= tol, "%s max abs error %.3g > %.1g" % (name, worst, tol)
    return worst


def check_bf16_exact(got, ref, name):
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    bad = got != ref
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d bf16 outputs differ; first at %s: got %04x want %04x (%d ulp)"
                             % (name, int(bad.sum()), bad.size, tuple(i), int(got[tuple(i)]),
                                int(ref[tuple(i)]), int(ulp_dist(got[tuple(i)], ref[tuple(i)]))))


def check_bf16_tol(got, ref, T, name, rel=COEF_TOL):
    """<= 1 ulp, or |d| <= ulp(y_ref) + rel * T where T = sum |terms|.
    T may be a callable returning that array; it is then evaluated only when
    some output is more than 1 ulp off.
    Returns (count within 1 ulp but not exact, count using the floor clause)."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    du = ulp_dist(got, ref)
    far = du > 1
    n_floor = 0
    if far.any():
        if callable(T):
            T = T()
        g = bf16_f64(got[far])
        r = bf16_f64(ref[far])
        lim = bf16_ulp(r) + rel * np.asarray(T, np.float64)[far]
        ok = np.abs(g - r) <= lim
        if not ok.all():
            k = np.argwhere(far)[np.argmax(~ok)]
            raise AssertionError("%s: %d bf16 outputs beyond tolerance; e.g. at %s got %r want %r (T=%r)"
                                 % (name, int((~ok).sum()), tuple(k), float(bf16_f64(got[tuple(k)])),
                                    float(bf16_f64(ref[tuple(k)])), float(np.asarray(T)[tuple(k)])))
        n_floor = int(far.sum())
    return int((du == 1).sum()), n_floor


def pre_terms(R_bits, pre):
    """sum_k |pre_k R_k| per output of hc_pre: [n, d]."""
    return np.einsum("nk,nkd->nd", np.abs(pre), np.abs(bf16_f64(R_bits)))


def post_terms(x_bits, R_bits, post, comb):
    """|post_k x| + sum_j |comb_jk R_j| per output of hc_post: [n, hc, d]."""
    X = np.abs(bf16_f64(x_bits))
    Rv = np.abs(bf16_f64(R_bits))
    return np.abs(post)[:, :, None] * X[:, None, :] + np.einsum("njk,njd->nkd", np.abs(comb), Rv)


def check_norm(got, ref, name, max_frac=1e-6):
    """RMSNorm outputs: NaN exactly where the oracle has NaN, every other
    output within 1 bf16 ulp, and at most max_frac of them (plus two) off by
    that ulp: only the order of the double sum of squares differs, which
    moves r by at most an ulp of double.  Returns the 1-ulp count."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    gn = (got & 0x7FFF) > 0x7F80
    rn = (ref & 0x7FFF) > 0x7F80
    assert (gn == rn).all(), "%s: NaN at %d outputs, oracle %d" % (name, int(gn.sum()), int(rn.sum()))
    du = ulp_dist(got[~rn], ref[~rn])
    worst = int(du.max()) if du.size else 0
    assert worst <= 1, "%s: an output %d bf16 ulp off" % (name, worst)
    off = int((du == 1).sum())
    assert off <= max_frac * du.size + 2, "%s: %d of %d outputs 1 ulp off" % (name, off, du.size)
    return off
