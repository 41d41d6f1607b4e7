"""libhc: hyper-connection residual-stream mixing on MI355X (gfx950).

Thin Python binding over the C-ABI in ``include/hc.h``: each function here
has the name of the C entry point it calls, checks dtypes, shapes, devices
and contiguity, allocates outputs with torch (device memory only), passes
raw pointers and torch's current HIP stream, and raises ``HCError`` on a
non-zero status.  Every step of the computation runs in the HIP kernels of
``libhc.so``; there is no fallback of any kind -- without the built library
or a GPU tensor every call raises.

Tensor shapes follow the pages' Block methods ("Mix projection" page):
residual ``R`` [..., hc, d] bf16, sublayer output ``x`` / input ``h``
[..., d] bf16, ``hc_fn`` [M, hc*d] fp32, ``hc_scale`` [3], ``hc_base``
[M] fp32, mixes [..., M], pre/post [..., hc], comb [..., hc, hc] fp32, where
M = (2 + hc) * hc (24 at the model's hc = 4).  hc is read from ``R`` and may
be 1..8; the packed-weight calls take hc = 4 only.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "HCError", "load", "lib_path", "hc_mixes", "hc_split_sinkhorn", "hc_pre", "hc_post",
    "hc_rmsnorm", "hc_pre_norm", "hc_fused_mix_pre", "hc_fused_mix_pre_norm", "hc_fused_mix_pre_noalloc", "hc_post_mix_pre", "hc_pack_weights", "hc_diag_scale", "hc_fused_workspace_bytes",
    "hc_post_backward", "hc_mix_pre_backward", "hc_backward_workspace_bytes",
    "Workspace", "workspace_status", "probe_stream", "check_workspace", "noalloc_status", "debug_force_timeout",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libhc.so")
_lib = None

HC_MIX = 24


class HCError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().hc_status_str(status).decode()
        super().__init__("%s failed: %s (status %d)" % (fn, msg, status))
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def use_library(path: str) -> None:
    """Load the library from `path` instead of libhc.so: the phase-tracing
    build (libhc_trace.so, ``python -m hyper_connection_residual_02_amd.build
    --phase-trace``).  Call it before the first library call."""
    global _LIB_PATH
    if _lib is not None and os.path.abspath(path) != os.path.abspath(_LIB_PATH):
        raise RuntimeError("the library is loaded already (%s)" % _LIB_PATH)
    _LIB_PATH = path


def trace_library_path() -> str:
    return os.path.join(_HERE, "libhc_trace.so")


def load():
    """Load libhc.so (built in-tree by ``hyper_connection_residual_02_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libhc.so is not built (%s); run "
                          "`python -m hyper_connection_residual_02_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_float, ctypes.c_size_t)
    sig = {
        "hc_mixes": [P, P, P, I64, I32, I32, F32, P, SZ, P],
        "hc_split_sinkhorn": [P, P, P, P, P, P, I64, I32, I32, F32, P],
        "hc_pre": [P, P, P, I64, I32, I32, P],
        "hc_rmsnorm": [P, P, P, I64, I32, F32, P],
        "hc_pre_norm": [P, P, P, P, P, I64, I32, I32, F32, P],
        "hc_post": [P, P, P, P, P, I64, I32, I32, P],
        "hc_fused_mix_pre": [P, P, P, P, P, P, P, P, P, P, SZ, I64, I32, I32, I32, F32, F32, P],
        "hc_fused_mix_pre_norm": [P, P, P, P, P, P, P, P, P, P, P, P, SZ, I64, I32, I32, I32, F32, F32, P],
        "hc_post_mix_pre": [P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, I64, I32, I32, I32, F32, F32, P],
        "hc_pack_weights": [P, P, SZ, I32, I32, P],
        "hc_fused_mix_pre_packed": [P, P, SZ, P, P, P, P, P, P, P, P, SZ, I64, I32, I32, I32, F32, F32, P],
        "hc_diag_scale": [P, P, P, I64, I32, P],
        "hc_probe_stream": [P, P, SZ, I32, P],
        "hc_fused_mix_pre_noalloc": [P, P, P, P, P, P, P, P, P, I64, I32, I32, I32, F32, F32, P],
        "hc_post_backward": [P, P, P, P, P, P, P, P, I64, I32, I32, P],
        "hc_mix_pre_backward": [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, I64, I32, I32, I32, F32, F32, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.hc_fused_workspace_bytes.argtypes = [I64, I32, I32]
    lib.hc_fused_workspace_bytes.restype = SZ
    lib.hc_packed_weights_bytes.argtypes = [I32, I32]
    lib.hc_packed_weights_bytes.restype = SZ
    lib.hc_workspace_status.argtypes = [P, SZ, ctypes.c_int]
    lib.hc_workspace_status.restype = ctypes.c_int
    lib.hc_noalloc_status.argtypes = [ctypes.c_int]
    lib.hc_noalloc_status.restype = ctypes.c_int
    lib.hc_debug_force_timeout.argtypes = [ctypes.c_int]
    lib.hc_debug_force_timeout.restype = ctypes.c_int
    lib.hc_phase_trace.argtypes = [P, SZ]
    lib.hc_phase_trace.restype = ctypes.c_int
    lib.hc_backward_workspace_bytes.argtypes = [I64, I32, I32]
    lib.hc_backward_workspace_bytes.restype = SZ
    lib.hc_scratch_bytes.argtypes = []
    lib.hc_scratch_bytes.restype = SZ
    lib.hc_status_str.argtypes = [ctypes.c_int]
    lib.hc_status_str.restype = ctypes.c_char_p
    lib.hc_version.argtypes = []
    lib.hc_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---------------------------------------------------------------- helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(t: torch.Tensor, name: str, dtype, dev=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU device (libhc has no CPU path)" % name)
    if dev is not None and t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _call(fn: str, *args):
    st = getattr(load(), fn)(*args)
    if st != 0:
        raise HCError(fn, st)


def probe_stream(src: torch.Tensor, dst: torch.Tensor | None = None, wg_per_cu: int = 0) -> None:
    """The bandwidth probe: copy src into dst (same size), or read src when
    dst is None, with the streaming kernels' access pattern, on wg_per_cu
    workgroups per compute unit (0: two)."""
    dev = src.device
    if src.device.type != "cuda" or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if dst is not None and (dst.device != dev or not dst.is_contiguous()
                            or dst.numel() * dst.element_size() != nbytes):
        raise ValueError("dst must be a contiguous GPU tensor of src's size, on its device")
    with torch.cuda.device(dev):
        _call("hc_probe_stream", _ptr(src), _ptr(dst), nbytes, int(wg_per_cu), _stream(dev))


def phase_trace(words: int):
    """The phase tables of the persistent projection kernel's last launch
    (phase-tracing build only, see use_library): a uint64 numpy array of up
    to `words` words, [1024 workgroups][8 waves][7]: the s_memrealtime ticks
    (100 MHz) of phases 0..5, then the round loop's tick count; then
    [1024 workgroups][4] clock stamps: entry, end of start-up, start of the
    round loop, end (include/hc.h, hc_phase_trace).  Synchronises."""
    import numpy as np
    out = np.zeros(int(words), dtype=np.uint64)
    torch.cuda.synchronize()
    r = load().hc_phase_trace(out.ctypes.data, out.size)
    if r < 0:
        raise HCError("hc_phase_trace", r)
    return out[:r]


def hc_fused_workspace_bytes(n: int, hc: int, d: int) -> int:
    """Workspace bytes hc_mixes / hc_fused_mix_pre need (host-only query)."""
    return int(load().hc_fused_workspace_bytes(int(n), int(hc), int(d)))


class Workspace:
    """A reusable, 256-byte aligned device workspace that grows on demand.

    Calls that may run at the same time (on different streams) each need a
    workspace of their own.  When one is used on a stream other than the one
    its memory was allocated on, the memory is recorded on that stream, so
    that growing it never hands memory still in use back to the allocator."""

    def __init__(self, device=None):
        self.device = torch.device(device) if device is not None else None
        self._buf = None
        self._off = 0
        self._alloc_stream = None
        self.nbytes = 0

    def get(self, nbytes: int, device: torch.device):
        cur = torch.cuda.current_stream(device)
        if self._buf is None or nbytes > self.nbytes or self._buf.device != device:
            self._buf = torch.empty(int(nbytes) + 256, dtype=torch.uint8, device=device)
            self._off = (-self._buf.data_ptr()) % 256
            self._alloc_stream = cur
            self.nbytes = int(nbytes)
        elif cur != self._alloc_stream:
            self._buf.record_stream(cur)
        return ctypes.c_void_p(self._buf.data_ptr() + self._off), self.nbytes

    def status(self, clear: bool = True) -> int:
        """hc_workspace_status of this workspace (0, or -10 when a call on it
        gave up a bounded wait); synchronise with its calls first."""
        if self._buf is None:
            return 0
        with torch.cuda.device(self._buf.device):
            return int(load().hc_workspace_status(ctypes.c_void_p(self._buf.data_ptr() + self._off),
                                                  self.nbytes, int(bool(clear))))


# default workspaces, one per (device, stream): calls on different streams
# may run at the same time, so they never share one
_default_ws = {}


def _workspace(ws, nbytes, dev):
    if ws is None:
        key = (str(dev), torch.cuda.current_stream(dev).cuda_stream)
        ws = _default_ws.setdefault(key, Workspace())
    return ws.get(max(int(nbytes), 256), dev)


def workspace_status(workspace: Workspace | None = None, device=None, clear: bool = True) -> int:
    """0 if no call on ``workspace`` (default: every default workspace of
    ``device``) gave up a bounded wait since the last clear, else -10
    (HC_ERR_TIMEOUT).  Synchronise with the calls first."""
    if workspace is not None:
        return workspace.status(clear)
    dev = str(torch.device(device if device is not None else "cuda"))
    worst = 0
    for (d, _), ws in list(_default_ws.items()):
        if device is None or d == dev:
            worst = min(worst, ws.status(clear))
    return worst


def check_workspace(workspace: Workspace | None = None, device=None):
    """Raise HCError when workspace_status reports a failed call."""
    st = workspace_status(workspace, device, clear=True)
    if st != 0:
        raise HCError("hc_workspace_status", st)


def noalloc_status(device=None, clear: bool = True) -> int:
    """hc_noalloc_status: the same for the static scratch of the no-alloc call."""
    with torch.cuda.device(torch.device(device if device is not None else "cuda")):
        return int(load().hc_noalloc_status(int(bool(clear))))


def debug_force_timeout(calls: int = 1):
    """Diagnostics: the next ``calls`` launches of the waiting kernels on this
    thread give up at their first exchange (hc_debug_force_timeout)."""
    _call("hc_debug_force_timeout", int(calls))


def _streams(R: torch.Tensor) -> int:
    """Stream count hc of a residual [..., hc, d] (libhc serves 1..8)."""
    if R.dim() < 2:
        raise ValueError("R must have shape [..., hc, d], got %s" % (tuple(R.shape),))
    return int(R.shape[-2])


def _lead(R: torch.Tensor, hc: int, name="R"):
    if R.dim() < 2 or R.shape[-2] != hc:
        raise ValueError("%s must have shape [..., %d, d], got %s" % (name, hc, tuple(R.shape)))
    lead = tuple(R.shape[:-2])
    n = 1
    for s in lead:
        n *= s
    return lead, n, R.shape[-1]


# ------------------------------------------------------------------- ops

def hc_mixes(R: torch.Tensor, hc_fn: torch.Tensor, norm_eps: float = 1e-20,
             out: torch.Tensor | None = None, workspace: Workspace | None = None) -> torch.Tensor:
    """mixes = (flatten(R) @ hc_fn^T) / RMS(flatten(R)); [..., (2+hc)*hc] fp32,
    hc = R.shape[-2] (1..8)."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    _check(hc_fn, "hc_fn", torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(hc_fn.shape) != (M, hc * d):
        raise ValueError("hc_fn must be [%d, %d], got %s" % (M, hc * d, tuple(hc_fn.shape)))
    if out is None:
        out = torch.empty(*lead, M, dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, dev)
    # other stream counts run a plain kernel that takes no workspace
    wp, wb = _workspace(workspace, hc_fused_workspace_bytes(n, hc, d), dev) if hc == 4 else (None, 0)
    with torch.cuda.device(dev):
        _call("hc_mixes", _ptr(R), _ptr(hc_fn), _ptr(out), n, hc, d, float(norm_eps), wp, wb,
              _stream(dev))
    return out


def hc_split_sinkhorn(mixes: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                      hc_mult: int = 4, sinkhorn_iters: int = 20, eps: float = 1e-6):
    """(pre [...,hc], post [...,hc], comb [...,hc,hc]) from mixes [..., (2+hc)*hc]."""
    dev = mixes.device
    _check(mixes, "mixes", torch.float32)
    _check(hc_scale, "hc_scale", torch.float32, dev)
    _check(hc_base, "hc_base", torch.float32, dev)
    M = (2 + hc_mult) * hc_mult
    if mixes.shape[-1] != M:
        raise ValueError("mixes must be [..., %d]" % M)
    lead = tuple(mixes.shape[:-1])
    n = mixes.numel() // M
    pre = torch.empty(*lead, hc_mult, dtype=torch.float32, device=dev)
    post = torch.empty(*lead, hc_mult, dtype=torch.float32, device=dev)
    comb = torch.empty(*lead, hc_mult, hc_mult, dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _call("hc_split_sinkhorn", _ptr(mixes), _ptr(hc_scale), _ptr(hc_base), _ptr(pre),
              _ptr(post), _ptr(comb), n, hc_mult, int(sinkhorn_iters), float(eps), _stream(dev))
    return pre, post, comb


def hc_pre(R: torch.Tensor, pre: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """h = bf16(sum_k pre[..., k] * R[..., k, :]); [..., d] bf16."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    _check(pre, "pre", torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(pre.shape) != lead + (hc,):
        raise ValueError("pre must be %s" % (lead + (hc,),))
    if out is None:
        out = torch.empty(*lead, d, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, dev)
    with torch.cuda.device(dev):
        _call("hc_pre", _ptr(R), _ptr(pre), _ptr(out), n, hc, d, _stream(dev))
    return out


def hc_rmsnorm(h: torch.Tensor, gamma: torch.Tensor, norm_eps: float = 1e-20,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """y = bf16(h * gamma / sqrt(mean(h^2) + norm_eps)) over the last axis; [..., d] bf16."""
    dev = h.device
    _check(h, "h", torch.bfloat16)
    _check(gamma, "gamma", torch.float32, dev)
    d = h.shape[-1]
    n = h.numel() // d if d else 0
    if tuple(gamma.shape) != (d,):
        raise ValueError("gamma must be (%d,)" % d)
    if out is None:
        out = torch.empty_like(h)
    _check(out, "out", torch.bfloat16, dev)
    if tuple(out.shape) != tuple(h.shape):
        raise ValueError("out must be %s" % (tuple(h.shape),))
    with torch.cuda.device(dev):
        _call("hc_rmsnorm", _ptr(h), _ptr(gamma), _ptr(out), n, d, norm_eps, _stream(dev))
    return out


def hc_pre_norm(R: torch.Tensor, pre: torch.Tensor, gamma: torch.Tensor, norm_eps: float = 1e-20,
                want_h: bool = False, out: torch.Tensor | None = None):
    """hc_pre then hc_rmsnorm in one pass over R: returns y, or (y, h) with ``want_h``."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    _check(pre, "pre", torch.float32, dev)
    _check(gamma, "gamma", torch.float32, dev)
    hc = _streams(R)
    lead, n, d = _lead(R, hc)
    if tuple(pre.shape) != lead + (hc,):
        raise ValueError("pre must be %s" % (lead + (hc,),))
    if tuple(gamma.shape) != (d,):
        raise ValueError("gamma must be (%d,)" % d)
    if out is None:
        out = torch.empty(*lead, d, dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, dev)
    h = torch.empty(*lead, d, dtype=torch.bfloat16, device=dev) if want_h else None
    with torch.cuda.device(dev):
        _call("hc_pre_norm", _ptr(R), _ptr(pre), _ptr(gamma), _ptr(h),
              _ptr(out), n, hc, d, norm_eps, _stream(dev))
    return (out, h) if want_h else out


def hc_post(x: torch.Tensor, R: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """R'[..., k, :] = bf16(post[..., k] x + sum_j comb[..., j, k] R[..., j, :]).
    ``out`` may be ``R`` itself (in place)."""
    dev = R.device
    _check(x, "x", torch.bfloat16, dev)
    _check(R, "R", torch.bfloat16)
    _check(post, "post", torch.float32, dev)
    _check(comb, "comb", torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(x.shape) != lead + (d,) or tuple(post.shape) != lead + (hc,) or \
            tuple(comb.shape) != lead + (hc, hc):
        raise ValueError("shape mismatch among x, R, post, comb")
    if out is None:
        out = torch.empty_like(R)
    _check(out, "out", torch.bfloat16, dev)
    with torch.cuda.device(dev):
        _call("hc_post", _ptr(x), _ptr(R), _ptr(post), _ptr(comb), _ptr(out), n, hc, d,
              _stream(dev))
    return out


def hc_pack_weights(hc_fn: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """The projection weights split once into the kernels' bf16 pieces
    (uint8 tensor); pass it as ``packed=`` to hc_fused_mix_pre."""
    dev = hc_fn.device
    _check(hc_fn, "hc_fn", torch.float32)
    hc = 4
    if hc_fn.dim() != 2 or hc_fn.shape[0] != HC_MIX or hc_fn.shape[1] % hc:
        raise ValueError("hc_fn must be [24, 4*d]")
    d = hc_fn.shape[1] // hc
    nb = int(load().hc_packed_weights_bytes(hc, d))
    if nb == 0:
        raise HCError("hc_pack_weights", -4)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=dev)
    _check(out, "out", torch.uint8, dev)
    with torch.cuda.device(dev):
        _call("hc_pack_weights", _ptr(hc_fn), _ptr(out), out.numel(), hc, d, _stream(dev))
    return out


def hc_fused_mix_pre(R: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor,
                     hc_base: torch.Tensor, sinkhorn_iters: int = 20, hc_eps: float = 1e-6,
                     norm_eps: float = 1e-20, want_pre: bool = True, want_mixes: bool = False,
                     workspace: Workspace | None = None, out=None, packed: torch.Tensor | None = None):
    """hc_mixes + hc_split_sinkhorn + hc_pre in one pass over R.
    Returns (h, pre or None, post, comb, mixes or None).  ``out`` may be a
    dict of preallocated outputs (keys h, pre, post, comb, mixes).  With
    ``packed`` (from hc_pack_weights(hc_fn)) the weights are not split again;
    hc_fn is then only checked for shape."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    for t, nm in ((hc_fn, "hc_fn"), (hc_scale, "hc_scale"), (hc_base, "hc_base")):
        _check(t, nm, torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(hc_fn.shape) != (M, hc * d):
        raise ValueError("hc_fn must be [%d, %d]" % (M, hc * d))
    o = dict(out or {})
    h = o.get("h") if o.get("h") is not None else torch.empty(*lead, d, dtype=torch.bfloat16, device=dev)
    post = o.get("post") if o.get("post") is not None else torch.empty(*lead, hc, dtype=torch.float32, device=dev)
    comb = o.get("comb") if o.get("comb") is not None else torch.empty(*lead, hc, hc, dtype=torch.float32, device=dev)
    pre = o.get("pre")
    if pre is None and want_pre:
        pre = torch.empty(*lead, hc, dtype=torch.float32, device=dev)
    mixes = o.get("mixes")
    if mixes is None and want_mixes:
        mixes = torch.empty(*lead, M, dtype=torch.float32, device=dev)
    wp, wb = _workspace(workspace, hc_fused_workspace_bytes(n, hc, d), dev)
    with torch.cuda.device(dev):
        if packed is not None:
            _check(packed, "packed", torch.uint8, dev)
            _call("hc_fused_mix_pre_packed", _ptr(R), _ptr(packed), packed.numel(), _ptr(hc_scale),
                  _ptr(hc_base), _ptr(h), _ptr(pre), _ptr(post), _ptr(comb), _ptr(mixes), wp, wb, n, hc, d,
                  int(sinkhorn_iters), float(hc_eps), float(norm_eps), _stream(dev))
        else:
            _call("hc_fused_mix_pre", _ptr(R), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), _ptr(h),
                  _ptr(pre), _ptr(post), _ptr(comb), _ptr(mixes), wp, wb, n, hc, d,
                  int(sinkhorn_iters), float(hc_eps), float(norm_eps), _stream(dev))
    return h, pre, post, comb, mixes


def hc_fused_mix_pre_norm(R: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor,
                          hc_base: torch.Tensor, gamma: torch.Tensor, sinkhorn_iters: int = 20,
                          hc_eps: float = 1e-6, norm_eps: float = 1e-20, want_h: bool = False,
                          want_pre: bool = True, want_mixes: bool = False,
                          workspace: Workspace | None = None, out=None):
    """hc_fused_mix_pre followed by the pre-sublayer RMSNorm of h.
    Returns (y, h or None, pre or None, post, comb, mixes or None).  ``out``
    may be a dict of preallocated outputs (keys y, h, pre, post, comb, mixes)."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    for t, nm in ((hc_fn, "hc_fn"), (hc_scale, "hc_scale"), (hc_base, "hc_base"), (gamma, "gamma")):
        _check(t, nm, torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(hc_fn.shape) != (M, hc * d):
        raise ValueError("hc_fn must be [%d, %d]" % (M, hc * d))
    if tuple(gamma.shape) != (d,):
        raise ValueError("gamma must be (%d,)" % d)
    o = dict(out or {})

    def get(key, want, shape, dtype):
        t = o.get(key)
        if t is None and want:
            t = torch.empty(*shape, dtype=dtype, device=dev)
        return t
    y = get("y", True, lead + (d,), torch.bfloat16)
    h = get("h", want_h, lead + (d,), torch.bfloat16)
    post = get("post", True, lead + (hc,), torch.float32)
    comb = get("comb", True, lead + (hc, hc), torch.float32)
    pre = get("pre", want_pre, lead + (hc,), torch.float32)
    mixes = get("mixes", want_mixes, lead + (M,), torch.float32)
    wp, wb = _workspace(workspace, hc_fused_workspace_bytes(n, hc, d), dev)
    with torch.cuda.device(dev):
        _call("hc_fused_mix_pre_norm", _ptr(R), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), _ptr(gamma),
              _ptr(h), _ptr(y), _ptr(pre), _ptr(post), _ptr(comb), _ptr(mixes), wp, wb, n, hc, d,
              int(sinkhorn_iters), float(hc_eps), float(norm_eps), _stream(dev))
    return y, h, pre, post, comb, mixes


def hc_fused_mix_pre_noalloc(R: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor,
                             hc_base: torch.Tensor, sinkhorn_iters: int = 20, hc_eps: float = 1e-6,
                             norm_eps: float = 1e-20, out=None):
    """hc_fused_mix_pre with the library's static scratch as its workspace:
    the C call allocates nothing.  ``out`` is a dict with the preallocated
    outputs h, post, comb (required) and pre, mixes (optional), so that this
    wrapper allocates nothing either.  Returns (h, pre, post, comb, mixes)."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    for t, nm in ((hc_fn, "hc_fn"), (hc_scale, "hc_scale"), (hc_base, "hc_base")):
        _check(t, nm, torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(hc_fn.shape) != (M, hc * d):
        raise ValueError("hc_fn must be [%d, %d]" % (M, hc * d))
    o = dict(out or {})
    for k in ("h", "post", "comb"):
        if o.get(k) is None:
            raise ValueError("out[%r] is required (this call allocates nothing)" % k)
    h, post, comb, pre, mixes = o["h"], o["post"], o["comb"], o.get("pre"), o.get("mixes")
    _check(h, "h", torch.bfloat16, dev)
    for t, nm, shape in ((post, "post", lead + (hc,)), (comb, "comb", lead + (hc, hc)),
                         (pre, "pre", lead + (hc,)), (mixes, "mixes", lead + (M,))):
        if t is not None:
            _check(t, nm, torch.float32, dev)
            if tuple(t.shape) != tuple(shape):
                raise ValueError("%s must be %s" % (nm, shape))
    if tuple(h.shape) != lead + (d,):
        raise ValueError("h must be %s" % (lead + (d,),))
    with torch.cuda.device(dev):
        _call("hc_fused_mix_pre_noalloc", _ptr(R), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), _ptr(h),
              _ptr(pre), _ptr(post), _ptr(comb), _ptr(mixes), n, hc, d, int(sinkhorn_iters), float(hc_eps),
              float(norm_eps), _stream(dev))
    return h, pre, post, comb, mixes


def hc_post_mix_pre(x: torch.Tensor, R: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
                    hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                    sinkhorn_iters: int = 20, hc_eps: float = 1e-6, norm_eps: float = 1e-20,
                    want_pre: bool = True, want_mixes: bool = False, workspace: Workspace | None = None,
                    out_R: torch.Tensor | None = None, out=None):
    """hc_post of one sublayer, then hc_fused_mix_pre of the next on its
    output.  Returns (R_out, h, pre or None, post, comb, mixes or None);
    ``out_R`` may be R itself (in place)."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    _check(x, "x", torch.bfloat16, dev)
    _check(post, "post", torch.float32, dev)
    _check(comb, "comb", torch.float32, dev)
    for t, nm in ((hc_fn, "hc_fn"), (hc_scale, "hc_scale"), (hc_base, "hc_base")):
        _check(t, nm, torch.float32, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(x.shape) != tuple(lead) + (d,):
        raise ValueError("x must be %s" % ((*lead, d),))
    if tuple(hc_fn.shape) != (M, hc * d):
        raise ValueError("hc_fn must be [%d, %d]" % (M, hc * d))
    if out_R is None:
        out_R = torch.empty_like(R)
    _check(out_R, "out_R", torch.bfloat16, dev)
    o = dict(out or {})
    h = o.get("h") if o.get("h") is not None else torch.empty(*lead, d, dtype=torch.bfloat16, device=dev)
    post2 = o.get("post") if o.get("post") is not None else torch.empty(*lead, hc, dtype=torch.float32, device=dev)
    comb2 = o.get("comb") if o.get("comb") is not None else torch.empty(*lead, hc, hc, dtype=torch.float32, device=dev)
    pre2 = o.get("pre")
    if pre2 is None and want_pre:
        pre2 = torch.empty(*lead, hc, dtype=torch.float32, device=dev)
    mixes = o.get("mixes")
    if mixes is None and want_mixes:
        mixes = torch.empty(*lead, M, dtype=torch.float32, device=dev)
    wp, wb = _workspace(workspace, hc_fused_workspace_bytes(n, hc, d), dev)
    with torch.cuda.device(dev):
        _call("hc_post_mix_pre", _ptr(x), _ptr(R), _ptr(post), _ptr(comb), _ptr(out_R), _ptr(hc_fn),
              _ptr(hc_scale), _ptr(hc_base), _ptr(h), _ptr(pre2), _ptr(post2), _ptr(comb2), _ptr(mixes),
              wp, wb, n, hc, d, int(sinkhorn_iters), float(hc_eps), float(norm_eps), _stream(dev))
    return out_R, h, pre2, post2, comb2, mixes


def hc_diag_scale(h: torch.Tensor, D: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """x = bf16(h * D) with D [d] bf16: the chained-stack stand-in sublayer."""
    dev = h.device
    _check(h, "h", torch.bfloat16)
    _check(D, "D", torch.bfloat16, dev)
    d = h.shape[-1]
    if tuple(D.shape) != (d,):
        raise ValueError("D must be [%d]" % d)
    n = h.numel() // d
    if out is None:
        out = torch.empty_like(h)
    _check(out, "out", torch.bfloat16, dev)
    with torch.cuda.device(dev):
        _call("hc_diag_scale", _ptr(h), _ptr(D), _ptr(out), n, d, _stream(dev))
    return out


# ------------------------------------------------------------- backward

def hc_backward_workspace_bytes(n: int, hc: int, d: int) -> int:
    """Workspace bytes hc_mix_pre_backward needs (host-only query)."""
    return int(load().hc_backward_workspace_bytes(int(n), int(hc), int(d)))


def hc_post_backward(x: torch.Tensor, R: torch.Tensor, post: torch.Tensor, comb: torch.Tensor,
                     gRout: torch.Tensor):
    """Gradient through hc_post from dL/dR' (bf16, R's shape): returns
    (gx bf16 [..., d], gpost fp32 [..., 4], gcomb fp32 [..., 4, 4])."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    _check(x, "x", torch.bfloat16, dev)
    _check(gRout, "gRout", torch.bfloat16, dev)
    _check(post, "post", torch.float32, dev)
    _check(comb, "comb", torch.float32, dev)
    hc = _streams(R)
    lead, n, d = _lead(R, hc)
    if tuple(x.shape) != lead + (d,) or tuple(gRout.shape) != tuple(R.shape) or \
            tuple(post.shape) != lead + (hc,) or tuple(comb.shape) != lead + (hc, hc):
        raise ValueError("shape mismatch among x, R, post, comb, gRout")
    gx = torch.empty_like(x)
    gpost = torch.empty_like(post)
    gcomb = torch.empty_like(comb)
    with torch.cuda.device(dev):
        _call("hc_post_backward", _ptr(x), _ptr(R), _ptr(post), _ptr(comb), _ptr(gRout), _ptr(gx), _ptr(gpost),
              _ptr(gcomb), n, hc, d, _stream(dev))
    return gx, gpost, gcomb


def hc_mix_pre_backward(R: torch.Tensor, hc_fn: torch.Tensor, hc_scale: torch.Tensor, hc_base: torch.Tensor,
                        mixes: torch.Tensor, gh: torch.Tensor, gRout: torch.Tensor, gpost: torch.Tensor,
                        gcomb: torch.Tensor, sinkhorn_iters: int = 20, hc_eps: float = 1e-6,
                        norm_eps: float = 1e-20, want_gmixes: bool = False, workspace: Workspace | None = None):
    """The rest of the sublayer's gradient: returns (gR bf16 [..., 4, d],
    g_hc_fn fp32 [24, 4d], g_hc_scale fp32 [3], g_hc_base fp32 [24],
    gmixes fp32 [..., 24] or None)."""
    dev = R.device
    _check(R, "R", torch.bfloat16)
    for t, nm in ((hc_fn, "hc_fn"), (hc_scale, "hc_scale"), (hc_base, "hc_base"), (mixes, "mixes"),
                  (gpost, "gpost"), (gcomb, "gcomb")):
        _check(t, nm, torch.float32, dev)
    _check(gh, "gh", torch.bfloat16, dev)
    _check(gRout, "gRout", torch.bfloat16, dev)
    hc = _streams(R)
    M = (2 + hc) * hc
    lead, n, d = _lead(R, hc)
    if tuple(hc_fn.shape) != (M, hc * d) or tuple(mixes.shape) != lead + (M,) or tuple(gh.shape) != lead + (d,) \
            or tuple(gRout.shape) != tuple(R.shape) or tuple(gpost.shape) != lead + (hc,) \
            or tuple(gcomb.shape) != lead + (hc, hc):
        raise ValueError("shape mismatch among the backward's inputs")
    gR = torch.empty_like(R)
    gW = torch.empty_like(hc_fn)
    gs = torch.empty_like(hc_scale)
    gb = torch.empty_like(hc_base)
    gm = torch.empty_like(mixes) if want_gmixes else None
    wp, wb = _workspace(workspace, hc_backward_workspace_bytes(n, hc, d), dev)
    with torch.cuda.device(dev):
        _call("hc_mix_pre_backward", _ptr(R), _ptr(hc_fn), _ptr(hc_scale), _ptr(hc_base), _ptr(mixes), _ptr(gh),
              _ptr(gRout), _ptr(gpost), _ptr(gcomb), _ptr(gR), _ptr(gW), _ptr(gs), _ptr(gb), _ptr(gm), wp, wb, n,
              hc, d, int(sinkhorn_iters), float(hc_eps), float(norm_eps), _stream(dev))
    return gR, gW, gs, gb, gm
