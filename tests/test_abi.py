"""The C-ABI library loads, exports every entry point include/hc.h declares,
and its host-side checks return the documented status codes.  Every call
here is an error path or n == 0, so nothing is launched: these run without
a GPU."""
import ctypes
import os
import re

import pytest

import hyper_connection_residual_02_amd as hcl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")

OK, NULL, SHAPE, ALIGN, UNSUP, WS, ALIAS, VALUE = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"\b(hc_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hcl.lib_path()):
        import hyper_connection_residual_02_amd.build as b
        b.build(verbose=False)
    return hcl.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"hc_mixes", "hc_split_sinkhorn", "hc_pre", "hc_post", "hc_fused_mix_pre", "hc_post_mix_pre",
            "hc_fused_workspace_bytes", "hc_status_str", "hc_diag_scale"} <= set(names)
    for nm in names:
        assert hasattr(lib, nm), nm
    assert lib.hc_version().decode().count(".") == 2


def test_status_strings(lib):
    assert lib.hc_status_str(-10).decode().startswith("HC_ERR_TIMEOUT")
    for code in range(-11, 1):
        s = lib.hc_status_str(code).decode()
        assert s.startswith("HC_")
    assert lib.hc_status_str(-100).decode().startswith("HC_ERR_?")


A = 0x10000          # fake, aligned addresses: never dereferenced on error paths
B = 0x20000000
C = 0x40000000
D_ = 0x60000000
E = 0x70000000
F_ = 0x7C000000
P = ctypes.c_void_p


def post_call(lib, x=A, R=B, post=C, comb=D_, out=E, n=4, hc=4, d=64):
    return lib.hc_post(P(x), P(R), P(post), P(comb), P(out), n, hc, d, None)


def test_post_checks(lib):
    assert post_call(lib, n=0) == OK
    assert post_call(lib, n=-1) == SHAPE
    assert post_call(lib, d=60) == SHAPE
    assert post_call(lib, d=0) == SHAPE
    assert post_call(lib, hc=9) == UNSUP
    assert post_call(lib, hc=0) == UNSUP
    assert post_call(lib, hc=3, x=0) == NULL
    assert post_call(lib, hc=3, out=B + 16) == ALIAS
    assert post_call(lib, x=0) == NULL
    assert post_call(lib, comb=0) == NULL
    assert post_call(lib, R=B + 8) == ALIGN
    assert post_call(lib, out=E + 2) == ALIGN
    assert post_call(lib, out=B + 16) == ALIAS           # partial overlap with R
    assert post_call(lib, out=A) == ALIAS                # overlaps x
    assert post_call(lib, n=1 << 40) == SHAPE            # size bound


def test_pre_checks(lib):
    f = lambda R=A, p=B, h=C, n=4, hc=4, d=64: lib.hc_pre(P(R), P(p), P(h), n, hc, d, None)
    assert f(n=0) == OK
    assert f(hc=9) == UNSUP
    assert f(hc=8, h=0) == NULL
    assert f(hc=8, h=A + 4032) == ALIAS    # R spans 4 * 8 * 64 * 2 bytes at hc = 8
    assert f(d=12) == SHAPE
    assert f(h=0) == NULL
    assert f(p=B + 4) == ALIGN
    assert f(h=A + 64) == ALIAS


def test_norm_checks(lib):
    f = lambda h=A, g=B, y=C, n=4, d=64, eps=1e-20: lib.hc_rmsnorm(P(h), P(g), P(y), n, d, eps, None)
    assert f(n=0) == OK
    assert f(n=-1) == SHAPE
    assert f(d=12) == SHAPE
    assert f(d=32768 + 8) == UNSUP         # wider than the kernel holds
    assert f(n=0, d=32768 + 8) == UNSUP
    assert f(eps=-1.0) == VALUE
    assert f(eps=float("nan")) == VALUE
    assert f(h=0) == NULL
    assert f(g=0) == NULL
    assert f(y=0) == NULL
    assert f(g=B + 4) == ALIGN
    assert f(y=A + 256) == ALIAS            # h spans 4 * 64 * 2 bytes
    assert f(y=B + 128) == ALIAS            # gamma spans 64 * 4 bytes
    g = lambda R=A, p=B, gm=B + 4096, h=C, y=D_, n=4, hc=4, d=64, eps=1e-20: \
        lib.hc_pre_norm(P(R), P(p), P(gm), P(h), P(y), n, hc, d, eps, None)
    assert g(n=0) == OK
    assert g(n=0, h=0) == OK
    assert g(hc=9) == UNSUP
    assert g(hc=0) == UNSUP
    assert g(d=12) == SHAPE
    assert g(d=32768 + 8) == UNSUP
    assert g(eps=float("inf")) == VALUE
    assert g(R=0) == NULL
    assert g(p=0) == NULL
    assert g(gm=0) == NULL
    assert g(y=0) == NULL
    assert g(h=C + 8) == ALIGN
    assert g(y=D_ + 2) == ALIGN
    assert g(y=A + 1024) == ALIAS           # R spans 4 * 4 * 64 * 2 bytes
    assert g(h=A + 2032) == ALIAS
    assert g(y=C + 64) == ALIAS             # y overlaps h
    assert g(h=B + 4096 + 128) == ALIAS     # h overlaps gamma
    assert g(y=B + 16) == ALIAS             # y overlaps pre


def test_phase_trace_unsupported_in_the_library(lib):
    # libhc.so has no phase tracing compiled in: no device access, only the status
    buf = (ctypes.c_uint64 * 16)()
    lib.hc_phase_trace.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    assert lib.hc_phase_trace(ctypes.cast(buf, ctypes.c_void_p), 16) == UNSUP
    assert lib.hc_phase_trace(None, 16) == NULL
    assert lib.hc_phase_trace(None, 0) == UNSUP


def test_probe_checks(lib):
    f = lambda s=A, d=B, nb=4096, wg=0: lib.hc_probe_stream(P(s), P(d), nb, wg, None)
    assert f(nb=0) == OK
    assert f(nb=24) == SHAPE
    assert f(s=0) == NULL
    assert f(s=A + 8) == ALIGN
    assert f(d=B + 4) == ALIGN
    assert f(d=A + 1024) == ALIAS
    assert lib.hc_probe_stream(P(A), P(0), 24, 0, None) == SHAPE
    assert f(wg=33) == VALUE
    assert f(wg=-1) == VALUE


def test_split_checks(lib):
    f = lambda m=A, s=B, b=B + 64, pre=C, post=D_, comb=E, n=4, hc=4, it=20, eps=1e-6: \
        lib.hc_split_sinkhorn(P(m), P(s), P(b), P(pre), P(post), P(comb), n, hc, it, eps, None)
    assert f(n=0) == OK
    assert f(n=-3) == SHAPE
    assert f(it=0) == UNSUP
    assert f(hc=9) == UNSUP
    assert f(hc=0) == UNSUP
    assert f(hc=2, s=0) == NULL
    assert f(hc=2, comb=A + 96) == ALIAS   # mixes span 4 * 8 * 4 bytes at hc = 2
    assert f(eps=-1.0) == VALUE
    assert f(eps=float("nan")) == VALUE
    assert f(eps=float("inf")) == VALUE
    assert f(s=0) == NULL
    assert f(s=B + 2) == ALIGN
    assert f(pre=C + 4) == ALIGN
    assert f(post=C + 32) == ALIAS
    assert f(comb=A) == ALIAS


def test_fused_and_mixes_checks(lib):
    def f(R=A, W=B, s=C, b=C + 64, h=D_, pre=E, post=E + 4096, comb=E + 8192, mix=0, ws=F_,
          wsb=1 << 30, n=4, hc=4, d=64, it=20, eps=1e-6, neps=1e-20):
        return lib.hc_fused_mix_pre(P(R), P(W), P(s), P(b), P(h), P(pre), P(post), P(comb),
                                    P(mix), P(ws), wsb, n, hc, d, it, eps, neps, None)
    assert f(n=0) == OK
    assert f(d=48) == UNSUP            # d % 32 != 0: the projection cannot be tiled
    assert f(d=40) == SHAPE or f(d=40) == UNSUP
    assert f(d=67 * 32) == UNSUP       # no k in 1..5 with d % (32k) == 0 and d/(32k) <= 64
    assert f(it=0) == UNSUP
    assert f(eps=-1e-6) == VALUE
    assert f(neps=float("nan")) == VALUE
    assert f(R=0) == NULL
    assert f(h=0) == NULL
    assert f(ws=0) == WS
    assert f(ws=F_ + 128) == ALIGN     # workspace must be 256-byte aligned
    assert f(W=B + 8) == ALIGN
    assert f(wsb=16) == WS
    assert f(h=A) == ALIAS             # h overlaps R
    assert f(post=E) == ALIAS          # post overlaps pre
    assert f(mix=F_) == ALIAS          # mixes overlaps the workspace
    # other stream counts: the same checks on hc-sized buffers
    assert f(hc=9) == UNSUP
    assert f(hc=2, it=0) == UNSUP
    assert f(hc=2, ws=0) == WS
    assert f(hc=2, wsb=16) == WS
    assert f(hc=2, h=A) == ALIAS
    assert f(hc=2, d=60) == SHAPE

    def m(R=A, W=B, out=C, ws=F_, wsb=1 << 30, n=4, hc=4, d=64, neps=1e-20):
        return lib.hc_mixes(P(R), P(W), P(out), n, hc, d, neps, P(ws), wsb, None)
    assert m(n=0) == OK
    assert m(out=0) == NULL
    assert m(out=C + 4) == ALIGN
    assert m(out=A) == ALIAS
    assert m(wsb=0) == WS
    assert m(hc=9) == UNSUP
    assert m(hc=5, n=0) == OK
    assert m(hc=5, out=0) == NULL
    assert m(hc=5, out=A) == ALIAS


def test_fused_norm_checks(lib):
    GM, Y = 0x50000000, 0x58000000

    def f(R=A, W=B, s=C, b=C + 64, g=GM, h=D_, y=Y, pre=E, post=E + 4096, comb=E + 8192, mix=0, ws=F_,
          wsb=1 << 30, n=4, hc=4, d=64, it=20, eps=1e-6, neps=1e-20):
        return lib.hc_fused_mix_pre_norm(P(R), P(W), P(s), P(b), P(g), P(h), P(y), P(pre), P(post),
                                         P(comb), P(mix), P(ws), wsb, n, hc, d, it, eps, neps, None)
    assert f(n=0) == OK
    assert f(n=0, h=0) == OK
    assert f(n=-1) == SHAPE
    assert f(d=48) == UNSUP               # the projection cannot tile it
    assert f(d=32768 + 32) == UNSUP       # wider than the norm kernel holds
    assert f(hc=9) == UNSUP
    assert f(neps=-1.0) == VALUE
    assert f(it=0) == UNSUP
    assert f(g=0) == NULL
    assert f(y=0) == NULL
    assert f(h=0, y=0) == NULL
    assert f(R=0) == NULL
    assert f(g=GM + 4) == ALIGN
    assert f(y=Y + 2) == ALIGN
    assert f(y=A) == ALIAS                # y overlaps R
    assert f(y=D_ + 256) == ALIAS         # y overlaps h
    assert f(y=GM + 128) == ALIAS         # y overlaps gamma
    assert f(g=D_) == ALIAS               # gamma overlaps h (an output)
    assert f(g=E + 4096) == ALIAS         # gamma overlaps post
    assert f(y=F_ + 64) == ALIAS          # y inside the workspace
    assert f(h=0, y=A + 64) == ALIAS      # y standing in for h overlaps R
    assert f(h=0, ws=0) == WS
    assert f(hc=2, y=A) == ALIAS
    assert f(hc=2, g=0) == NULL
    assert f(hc=2, wsb=16) == WS


def test_post_mix_pre_checks(lib):
    H = 0x74000000

    def f(x=A, R=B, post=C, comb=C + 64, Ro=D_, W=E, s=E + 0x10000, b=E + 0x10040, h=H, pre=H + 0x1000,
          post2=H + 0x2000, comb2=H + 0x3000, mix=0, ws=F_, wsb=1 << 30, n=4, hc=4, d=64, it=20, eps=1e-6,
          neps=1e-20):
        return lib.hc_post_mix_pre(P(x), P(R), P(post), P(comb), P(Ro), P(W), P(s), P(b), P(h), P(pre),
                                   P(post2), P(comb2), P(mix), P(ws), wsb, n, hc, d, it, eps, neps, None)
    assert f(n=0) == OK
    assert f(hc=9) == UNSUP
    assert f(hc=3, Ro=B + 64) == ALIAS
    assert f(hc=3, ws=0) == WS
    assert f(hc=3, x=0) == NULL
    assert f(it=0) == UNSUP
    assert f(eps=-1.0) == VALUE
    assert f(x=0) == NULL
    assert f(comb=0) == NULL
    assert f(Ro=0) == NULL
    assert f(ws=0) == WS
    assert f(x=A + 8) == ALIGN
    assert f(Ro=B + 64) == ALIAS        # R_out overlaps R without being R
    assert f(h=B) == ALIAS              # an output over the residual
    assert f(post2=C) == ALIAS          # the next post over this sublayer's post
    assert f(comb2=H + 0x2008 - 8) == ALIAS   # comb_next over post_next


def test_packed_weights_checks(lib):
    assert lib.hc_packed_weights_bytes(4, 5120) == 32 * 4 * 5 * 5 * 64 * 16
    assert lib.hc_packed_weights_bytes(4, 64) == 0          # served by the cooperative kernel: no packed form
    assert lib.hc_packed_weights_bytes(3, 5120) == 0
    nb = lib.hc_packed_weights_bytes(4, 256)
    assert nb > 0

    def pk(W=A, out=B, nbytes=nb, hc=4, d=256):
        return lib.hc_pack_weights(P(W), P(out), nbytes, hc, d, None)
    assert pk(d=64) == UNSUP
    assert pk(hc=5) == UNSUP
    assert pk(d=40) == UNSUP or pk(d=40) == SHAPE
    assert pk(W=0) == NULL
    assert pk(out=B + 8) == ALIGN
    assert pk(nbytes=nb - 16) == WS
    assert pk(out=A + 1024) == ALIAS     # the packed form over the weights

    def f(R=A, pkd=B, nbytes=nb, s=C, b=C + 64, h=D_, pre=E, post=E + 4096, comb=E + 8192, mix=0, ws=F_,
          wsb=1 << 30, n=4, hc=4, d=256, it=20, eps=1e-6, neps=1e-20):
        return lib.hc_fused_mix_pre_packed(P(R), P(pkd), nbytes, P(s), P(b), P(h), P(pre), P(post), P(comb),
                                           P(mix), P(ws), wsb, n, hc, d, it, eps, neps, None)
    assert f(n=0) == OK
    assert f(pkd=0) == NULL
    assert f(nbytes=16) == WS
    assert f(d=64) == UNSUP
    assert f(hc=3) == UNSUP              # packed weights: four streams only
    assert f(h=B) == ALIAS               # h over the packed weights


def test_workspace_query(lib):
    assert lib.hc_fused_workspace_bytes(0, 4, 5120) == 0
    assert lib.hc_fused_workspace_bytes(16, 9, 5120) == 0
    # the projection's partial sums (8 segments of 15 + 2 floats per token),
    # then the mixes, then pre, each 256-byte aligned
    # partial sums, mixes, pre; calls of 1,024 tokens or more also hold the
    # weights split once (240 chunks x 6 KB at hc = 3, d = 5120)
    assert lib.hc_fused_workspace_bytes(16, 3, 5120) == 8704 + 1024 + 256
    assert lib.hc_fused_workspace_bytes(1024, 3, 5120) == 1024 * 8 * 17 * 4 + 1024 * 15 * 4 + 1024 * 3 * 4 + 240 * 6144
    assert lib.hc_fused_workspace_bytes(16, 4, 48) == 0
    assert lib.hc_fused_workspace_bytes(16, 4, 64) > 0
    assert lib.hc_fused_workspace_bytes(65536, 4, 5120) > 0


def test_noalloc_checks(lib):
    cap = lib.hc_scratch_bytes()
    assert cap == 16 << 20

    def call(n, hc=4, d=5120, R=A):
        return lib.hc_fused_mix_pre_noalloc(P(R), P(B), P(C), P(D_), P(E), None, P(F_), P(F_ + 4096), None,
                                            n, hc, d, 20, 1e-6, 1e-20, None)
    assert call(0) == OK
    assert call(-1) == SHAPE
    assert call(4, d=60) == SHAPE
    assert call(4, hc=9) == UNSUP
    big = 1
    while lib.hc_fused_workspace_bytes(big, 4, 5120) <= cap:
        big *= 2
    assert call(big) == -11                   # beyond the static scratch: rejected before any launch
    assert lib.hc_status_str(-11).decode().startswith("HC_ERR_SCRATCH")


def test_status_query_and_diagnostics_checks(lib):
    # argument checks only (no device memory is read on these paths)
    assert lib.hc_workspace_status(None, 4096, 1) == NULL
    assert lib.hc_workspace_status(P(A + 16), 4096, 1) == ALIGN
    assert lib.hc_workspace_status(P(A), 255, 1) == WS
    assert lib.hc_debug_force_timeout(-1) == VALUE
    assert lib.hc_debug_force_timeout(0) == OK


def test_backward_checks(lib):
    def post_b(n=4, hc=4, d=256, gx=E):
        return lib.hc_post_backward(P(A), P(B), P(C), P(D_), P(F_), P(gx), P(0x7E000000), P(0x7F000000), n, hc, d,
                                    None)
    assert post_b(n=0) == OK
    assert post_b(hc=3) == UNSUP
    assert post_b(d=60) == SHAPE
    assert post_b(gx=0) == NULL
    assert post_b(gx=E + 2) == ALIGN
    assert post_b(gx=B + 32) == ALIAS

    def mix_b(n=4, hc=4, d=256, iters=20, ws=0x78000000, wsb=1 << 24, gR=0x7A000000):
        return lib.hc_mix_pre_backward(P(A), P(B), P(C), P(C + 64), P(D_), P(E), P(F_), P(0x7E000000),
                                       P(0x7F000000), P(gR), P(0x7B000000), P(0x7C800000), P(0x7C900000), None,
                                       P(ws), wsb, n, hc, d, iters, 1e-6, 1e-20, None)
    assert mix_b(n=0) == OK
    assert mix_b(hc=2) == UNSUP
    assert mix_b(d=64) == UNSUP                  # d % 128 != 0
    assert mix_b(iters=65) == UNSUP and mix_b(iters=0) == UNSUP
    assert mix_b(ws=0) == WS
    assert mix_b(wsb=100) == WS
    assert mix_b(gR=0) == NULL
    assert mix_b(ws=0x78000010) == ALIGN
    assert mix_b(gR=B) == ALIAS
    assert lib.hc_backward_workspace_bytes(4, 4, 256) > 0
    assert lib.hc_backward_workspace_bytes(4, 3, 256) == 0


def test_diag_checks(lib):
    f = lambda h=A, Dp=B, x=C, n=4, d=64: lib.hc_diag_scale(P(h), P(Dp), P(x), n, d, None)
    assert f(n=0) == OK
    assert f(d=7) == SHAPE
    assert f(x=0) == NULL
    assert f(x=A) == ALIAS
    assert f(Dp=B + 2) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    R = torch.zeros(2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hcl.hc_pre(R, torch.zeros(2, 4))
