"""fp64 CPU oracle for hyper-connection residual mixing -- TEST INFRASTRUCTURE.

This package is the correctness reference the GPU library is checked against.
Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import it.  The product path (the GPU library and its Python binding)
never imports, links or calls anything here, and this package imports nothing
from the product.

The arithmetic lives in plain C (``hc_oracle.c``, double precision, OpenMP over
tokens); this module compiles it with gcc and wraps each function for numpy
arrays.  Every function follows a passage of the pages:

* ``mixes``          -- "Mix projection" page, the mix formula (RMS over the
                        flattened hc*d stream, eps 1e-20, projection to 24).
* ``split_sinkhorn`` -- "Reading weights" page, learned-pre formula and the
                        hc_split_sinkhorn kernel listing.
* ``pre``, ``post``  -- "Mix projection" page, Block.hc_pre / Block.hc_post.
* ``diag_scale``     -- the chained-stack workload's stand-in sublayer.
* ``post_backward``, ``pre_backward``, ``split_sinkhorn_backward``,
  ``mixes_backward``, ``backward`` -- the gradient of a scalar loss through
  the same steps (chain rule over the forward in reverse order; the pages
  give the forward only).
* ``round_bf16``     -- round-to-nearest-even from double to bf16.

bf16 tensors cross this interface as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hc_oracle.c")
_LIB = os.path.join(_HERE, "libhcoracle.so")
_lib = None

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/libhcoracle.so`` with gcc."""
    if force or not os.path.exists(_LIB) or \
            os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64, I32, F64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.hco_mixes.argtypes = [P, P, I64, I32, I32, F64, P]
    lib.hco_mixes.restype = None
    lib.hco_split_sinkhorn.argtypes = [P, P, P, I64, I32, I32, F64, P, P, P]
    lib.hco_split_sinkhorn.restype = ctypes.c_int
    lib.hco_pre.argtypes = [P, P, I64, I32, I32, P]
    lib.hco_pre.restype = None
    lib.hco_post.argtypes = [P, P, P, P, I64, I32, I32, P]
    lib.hco_post.restype = None
    lib.hco_diag_scale.argtypes = [P, P, I64, I32, P]
    lib.hco_diag_scale.restype = None
    lib.hco_rmsnorm.argtypes = [P, P, I64, I32, ctypes.c_double, P]
    lib.hco_rmsnorm.restype = None
    lib.hco_post_backward.argtypes = [P, P, P, P, P, I64, I32, I32, P, P, P, P]
    lib.hco_post_backward.restype = None
    lib.hco_pre_backward.argtypes = [P, P, P, I64, I32, I32, P, P]
    lib.hco_pre_backward.restype = None
    lib.hco_split_sinkhorn_backward.argtypes = [P, P, P, P, P, P, I64, I32, I32, F64, P, P, P]
    lib.hco_split_sinkhorn_backward.restype = ctypes.c_int
    lib.hco_mixes_backward.argtypes = [P, P, P, I64, I32, I32, F64, P, P]
    lib.hco_mixes_backward.restype = None
    lib.hco_round_bf16_array.argtypes = [P, I64, P]
    lib.hco_round_bf16_array.restype = None
    lib.hco_round_bf16.argtypes = [F64]
    lib.hco_round_bf16.restype = ctypes.c_uint16
    lib.hco_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.hco_bf16_to_double.restype = F64
    lib.hco_num_threads.argtypes = []
    lib.hco_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().hco_num_threads())


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(v: float) -> int:
    """Round one double to a bf16 bit pattern (nearest, ties to even)."""
    return int(_load().hco_round_bf16(float(v)))


def round_bf16_array(v) -> np.ndarray:
    """Round every double of ``v`` to a bf16 bit pattern (uint16, same shape)."""
    a, pa = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().hco_round_bf16_array(pa, a.size, out.ctypes.data)
    return out


def mixes(R_bits, W, norm_eps: float = 1e-20) -> np.ndarray:
    """R_bits uint16[n,hc,d], W float32[(2+hc)hc, hc*d] -> float64[n,(2+hc)hc]."""
    R, pR = _c(R_bits, np.uint16)
    n, hc, d = R.shape
    Wc, pW = _c(W, np.float32)
    M = (2 + hc) * hc
    assert Wc.shape == (M, hc * d), Wc.shape
    out = np.empty((n, M), dtype=np.float64)
    _load().hco_mixes(pR, pW, n, hc, d, float(norm_eps), out.ctypes.data)
    return out


def split_sinkhorn(mix, scale, base, hc: int = 4, iters: int = 20,
                   eps: float = 1e-6):
    """mix float[n,(2+hc)hc] -> (pre[n,hc], post[n,hc], comb[n,hc,hc]) float64."""
    m, pm = _c(mix, np.float64)
    n = m.shape[0]
    assert m.shape == (n, (2 + hc) * hc), m.shape
    s, ps = _c(scale, np.float32)
    b, pb = _c(base, np.float32)
    assert s.shape == (3,) and b.shape == ((2 + hc) * hc,)
    pre_ = np.empty((n, hc), dtype=np.float64)
    post_ = np.empty((n, hc), dtype=np.float64)
    comb_ = np.empty((n, hc, hc), dtype=np.float64)
    rc = _load().hco_split_sinkhorn(pm, ps, pb, n, hc, int(iters), float(eps),
                                    pre_.ctypes.data, post_.ctypes.data,
                                    comb_.ctypes.data)
    if rc != 0:
        raise ValueError("split_sinkhorn: unsupported hc=%d or iters=%d" % (hc, iters))
    return pre_, post_, comb_


def pre(R_bits, pre_w) -> np.ndarray:
    """R_bits uint16[n,hc,d], pre float[n,hc] -> h uint16[n,d]."""
    R, pR = _c(R_bits, np.uint16)
    n, hc, d = R.shape
    p, pp = _c(pre_w, np.float64)
    assert p.shape == (n, hc), p.shape
    h = np.empty((n, d), dtype=np.uint16)
    _load().hco_pre(pR, pp, n, hc, d, h.ctypes.data)
    return h


def post(x_bits, R_bits, post_w, comb) -> np.ndarray:
    """x uint16[n,d], R uint16[n,hc,d], post float[n,hc], comb float[n,hc,hc]
    -> R' uint16[n,hc,d]."""
    R, pR = _c(R_bits, np.uint16)
    n, hc, d = R.shape
    x, px = _c(x_bits, np.uint16)
    assert x.shape == (n, d), x.shape
    p, pp = _c(post_w, np.float64)
    cb, pc = _c(comb, np.float64)
    assert p.shape == (n, hc) and cb.shape == (n, hc, hc)
    out = np.empty((n, hc, d), dtype=np.uint16)
    _load().hco_post(px, pR, pp, pc, n, hc, d, out.ctypes.data)
    return out


def diag_scale(h_bits, D_bits) -> np.ndarray:
    """h uint16[n,d], D uint16[d] -> bf16(h * D) as uint16[n,d]."""
    h, ph = _c(h_bits, np.uint16)
    n, d = h.shape
    D, pD = _c(D_bits, np.uint16)
    assert D.shape == (d,)
    out = np.empty((n, d), dtype=np.uint16)
    _load().hco_diag_scale(ph, pD, n, d, out.ctypes.data)
    return out


def rmsnorm(h_bits, gamma, norm_eps: float = 1e-20) -> np.ndarray:
    """The pre-sublayer RMSNorm of the "Mix projection" page's Block.__init__
    (a reading: the pages print no formula) on hc_pre's bf16 output:
    y_c = bf16(h_c / sqrt(mean(h^2) + norm_eps) * gamma_c), in double, rounded
    once.  h_bits [..., d] uint16, gamma float32 [d]; returns uint16 [..., d]."""
    hb = np.ascontiguousarray(h_bits, dtype=np.uint16)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    d = hb.shape[-1]
    n = hb.size // d if d else 0
    out = np.empty_like(hb)
    if n:
        _load().hco_rmsnorm(hb.ctypes.data, g.ctypes.data, n, d, float(norm_eps), out.ctypes.data)
    return out


def fused(R_bits, W, scale, base, iters: int = 20, eps: float = 1e-6,
          norm_eps: float = 1e-20):
    """The whole collapse side for one sublayer: mixes, split/Sinkhorn, hc_pre.
    Returns (h uint16[n,d], pre, post, comb, mixes) with float64 coefficients."""
    R = np.asarray(R_bits, dtype=np.uint16)
    hc = R.shape[1]
    m = mixes(R, W, norm_eps)
    p, q, c = split_sinkhorn(m, scale, base, hc, iters, eps)
    h = pre(R, p)
    return h, p, q, c, m


# ------------------------------------------------------------------ backward

def post_backward(x_bits, R_bits, post_w, comb, gRout_bits):
    """Gradient through hc_post: (gx[n,d], gpost[n,hc], gcomb[n,hc,hc],
    gR[n,hc,d]) float64 from dL/dR' (bf16 patterns)."""
    R, pR = _c(R_bits, np.uint16)
    n, hc, d = R.shape
    x, px = _c(x_bits, np.uint16)
    g, pg = _c(gRout_bits, np.uint16)
    p, pp = _c(post_w, np.float64)
    cb, pc = _c(comb, np.float64)
    assert x.shape == (n, d) and g.shape == (n, hc, d)
    assert p.shape == (n, hc) and cb.shape == (n, hc, hc)
    gx = np.empty((n, d)); gp = np.empty((n, hc)); gc = np.empty((n, hc, hc))
    gR = np.empty((n, hc, d))
    _load().hco_post_backward(px, pR, pp, pc, pg, n, hc, d, gx.ctypes.data, gp.ctypes.data,
                              gc.ctypes.data, gR.ctypes.data)
    return gx, gp, gc, gR


def pre_backward(R_bits, pre_w, gh_bits):
    """Gradient through hc_pre: (gpre[n,hc], gR[n,hc,d]) float64 from dL/dh."""
    R, pR = _c(R_bits, np.uint16)
    n, hc, d = R.shape
    g, pg = _c(gh_bits, np.uint16)
    p, pp = _c(pre_w, np.float64)
    assert g.shape == (n, d) and p.shape == (n, hc)
    gpre = np.empty((n, hc)); gR = np.empty((n, hc, d))
    _load().hco_pre_backward(pR, pp, pg, n, hc, d, gpre.ctypes.data, gR.ctypes.data)
    return gpre, gR


def split_sinkhorn_backward(mix, scale, base, gpre, gpost, gcomb, hc: int = 4,
                            iters: int = 20, eps: float = 1e-6):
    """Gradient through the split + Sinkhorn: (gmixes[n,M], gscale[3],
    gbase[M], gscale_tok[n,3], gbase_tok[n,M]) float64; gscale and gbase are
    the per-token contributions summed over tokens in order."""
    m, pm = _c(mix, np.float64)
    n = m.shape[0]
    M = (2 + hc) * hc
    assert m.shape == (n, M)
    s, ps = _c(scale, np.float32)
    b, pb = _c(base, np.float32)
    gp, pgp = _c(gpre, np.float64)
    gq, pgq = _c(gpost, np.float64)
    gc, pgc = _c(gcomb, np.float64)
    assert gp.shape == (n, hc) and gq.shape == (n, hc) and gc.shape == (n, hc, hc)
    gm = np.empty((n, M)); gs = np.empty((n, 3)); gb = np.empty((n, M))
    rc = _load().hco_split_sinkhorn_backward(pm, ps, pb, pgp, pgq, pgc, n, hc, int(iters), float(eps),
                                             gm.ctypes.data, gs.ctypes.data, gb.ctypes.data)
    if rc != 0:
        raise ValueError("split_sinkhorn_backward: unsupported hc=%d or iters=%d" % (hc, iters))
    gsum = np.zeros(3); bsum = np.zeros(M)
    for t in range(n):
        gsum += gs[t]
        bsum += gb[t]
    return gm, gsum, bsum, gs, gb


def mixes_backward(R_bits, W, gmix, norm_eps: float = 1e-20):
    """Gradient through the mix formula: (gR[n,hc,d], gW[M,hc*d]) float64."""
    R, pR = _c(R_bits, np.uint16)
    n, hc, d = R.shape
    Wc, pW = _c(W, np.float32)
    M = (2 + hc) * hc
    g, pg = _c(gmix, np.float64)
    assert Wc.shape == (M, hc * d) and g.shape == (n, M)
    gR = np.empty((n, hc, d)); gW = np.empty((M, hc * d))
    _load().hco_mixes_backward(pR, pW, pg, n, hc, d, float(norm_eps), gR.ctypes.data, gW.ctypes.data)
    return gR, gW


def backward(R_bits, x_bits, W, scale, base, gRout_bits, gh_bits, iters: int = 20,
             eps: float = 1e-6, norm_eps: float = 1e-20, mix=None):
    """The whole gradient of one sublayer's mixing, given dL/dR' and dL/dh:
    the forward coefficients (from ``mix`` when given, else the oracle's own
    mixes), then hc_post's, hc_pre's, the split's and the projection's
    backward.  Returns a dict of float64 arrays: gR (the three shares
    summed), gR_post, gR_pre, gR_mix, gx, gpost, gcomb, gpre, gmixes, gW,
    gscale, gbase, and the coefficients pre, post, comb, mixes used."""
    R = np.asarray(R_bits, dtype=np.uint16)
    hc = R.shape[1]
    m = mixes(R, W, norm_eps) if mix is None else np.asarray(mix, dtype=np.float64)
    p, q, c = split_sinkhorn(m, scale, base, hc, iters, eps)
    gx, gpost, gcomb, gR_post = post_backward(x_bits, R, q, c, gRout_bits)
    gpre, gR_pre = pre_backward(R, p, gh_bits)
    gm, gs, gb, _, _ = split_sinkhorn_backward(m, scale, base, gpre, gpost, gcomb, hc, iters, eps)
    gR_mix, gW = mixes_backward(R, W, gm, norm_eps)
    return dict(gR=gR_post + gR_pre + gR_mix, gR_post=gR_post, gR_pre=gR_pre, gR_mix=gR_mix, gx=gx,
                gpost=gpost, gcomb=gcomb, gpre=gpre, gmixes=gm, gW=gW, gscale=gs, gbase=gb,
                pre=p, post=q, comb=c, mixes=m)
