"""Seeded synthetic inputs for the hyper-connection workloads.

This module holds no arithmetic of the method: it only draws random tensors
of the shapes and value distributions of the five workloads, so that the GPU
library and the CPU oracle can be fed the very same values.

Recipe (also stated in the design doc):

* every tensor has its own ``torch.Generator`` on the target device, seeded
  with ``seed * 1000 + stream`` where ``stream`` numbers the tensor
  (R=1, x=2, W=3, scale=4, base=5; chained layer l uses 100 + 10*l + {0..3});
* normals are drawn in float32 with ``torch.randn`` (Philox on GPU,
  mt19937 on CPU), uniforms with ``torch.rand`` mapped to [lo, hi);
* bf16 tensors are the float32 draws rounded to nearest-even by
  ``Tensor.to(torch.bfloat16)``;
* "N(0, s)" means standard deviation s.

The draws differ between CPU and GPU generators; every test feeds one tensor
to both sides, so only the distribution matters.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    hc: int
    d: int
    w_std: float
    s_lo: float
    s_hi: float
    b_std: float
    layers: int = 1
    d_lo: float = 0.5       # diagonal sublayer scale range (chained stack)
    d_hi: float = 1.5
    iters: int = 20
    hc_eps: float = 1e-6
    norm_eps: float = 1e-20
    seed: int = 0

    @property
    def n(self) -> int:
        return self.B * self.T

    @property
    def K(self) -> int:
        return self.hc * self.d

    @property
    def M(self) -> int:
        return (2 + self.hc) * self.hc


# The five workloads of the hot path (d = 5120 and hc = 4 are the model's
# dim and hc_mult; 24 x 20480 is the size of one mix projection).
WORKLOADS = {
    "tiny": Workload("tiny", 1, 16, 4, 64, 0.02, 0.5, 2.0, 1.0),
    "decode": Workload("decode", 64, 1, 4, 5120, 0.007, 0.5, 2.0, 1.0),
    "prefill": Workload("prefill", 1, 4096, 4, 5120, 0.007, 0.5, 2.0, 1.0),
    "large": Workload("large", 8, 8192, 4, 5120, 0.007, 0.5, 2.0, 1.0),
    "chained": Workload("chained", 4, 4096, 4, 5120, 0.007, 0.5, 20.0, 2.0,
                        layers=80),
}


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed) * 1000 + int(stream))
    return g


def randn(shape, std, device, seed, stream, dtype=torch.float32,
          chunk: int = 1 << 27) -> torch.Tensor:
    """N(0, std) draws in float32, cast to ``dtype``; generated in chunks of
    ``chunk`` elements so that huge bf16 tensors need little scratch."""
    g = _gen(device, seed, stream)
    numel = int(np.prod(shape))
    out = torch.empty(numel, dtype=dtype, device=device)
    for s in range(0, numel, chunk):
        e = min(numel, s + chunk)
        v = torch.randn(e - s, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            v.mul_(std)
        out[s:e] = v.to(dtype)
    return out.view(*shape)


def uniform(shape, lo, hi, device, seed, stream,
            dtype=torch.float32) -> torch.Tensor:
    g = _gen(device, seed, stream)
    v = torch.rand(*shape, generator=g, device=device, dtype=torch.float32)
    return (v * (hi - lo) + lo).to(dtype)


def make_inputs(w: Workload, device="cpu", seed=None, n_tokens=None):
    """Residual R bf16[B,T,hc,d], sublayer output x bf16[B,T,d], and one
    sublayer's parameters W fp32[M,K], scale fp32[3], base fp32[M].

    ``n_tokens`` (optional) overrides B*T with [1, n_tokens]."""
    seed = w.seed if seed is None else seed
    B, T = (w.B, w.T) if n_tokens is None else (1, int(n_tokens))
    R = randn((B, T, w.hc, w.d), 1.0, device, seed, 1, torch.bfloat16)
    x = randn((B, T, w.d), 1.0, device, seed, 2, torch.bfloat16)
    W, scale, base = make_params(w, device, seed, layer=None)
    return {"R": R, "x": x, "W": W, "scale": scale, "base": base}


def make_params(w: Workload, device="cpu", seed=None, layer=None):
    """(W, scale, base) for one sublayer.  ``layer`` selects a chained-stack
    layer's own parameters (None: the single-sublayer workloads)."""
    seed = w.seed if seed is None else seed
    off = 3 if layer is None else 100 + 10 * int(layer)
    W = randn((w.M, w.K), w.w_std, device, seed, off)
    scale = uniform((3,), w.s_lo, w.s_hi, device, seed, off + 1)
    base = randn((w.M,), w.b_std, device, seed, off + 2)
    return W, scale, base


def make_diag(w: Workload, layer: int, device="cpu", seed=None):
    """Chained-stack stand-in sublayer: a bf16 diagonal scale U(d_lo, d_hi)[d]."""
    seed = w.seed if seed is None else seed
    return uniform((w.d,), w.d_lo, w.d_hi, device, seed, 100 + 10 * int(layer) + 3,
                   torch.bfloat16)


def make_gamma(d: int, device="cpu", seed: int = 7, std: float = 0.25):
    """Pre-sublayer RMSNorm weight: fp32[d] drawn as 1 + N(0, std)."""
    return randn((d,), std, device, seed, 9).add_(1.0)


def sample_tokens(n: int, k: int, seed: int = 0) -> np.ndarray:
    """Sorted token indices for sampled checks: the first and last tokens,
    token boundaries of common tile sizes, and random ones."""
    rng = np.random.default_rng(12345 + seed)
    fixed = [0, 1, 15, 16, 63, 64, n // 2, n - 2, n - 1]
    picks = set(i for i in fixed if 0 <= i < n)
    if n > 0:
        picks.update(int(i) for i in rng.choice(n, size=min(n, k), replace=False))
    return np.array(sorted(picks), dtype=np.int64)


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (copied to host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(b: np.ndarray, device="cpu") -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor."""
    a = np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a.copy()).view(torch.bfloat16).to(device)
