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
