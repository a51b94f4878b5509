"""Seeded synthetic inputs for the FAVOR+ forward pass.

This module is shared by the tests, ``bench.py`` and ``__graft_entry__`` and
holds none of the method's arithmetic: it only draws Gaussian Q, K, V of the
workload shapes, applies the caller-side d^-1/4 pre-scale and the optional
per-head mean offsets, and casts to the input dtype (fp32 or bf16 with
round-to-nearest-even).  The projection W is not drawn here.

The workloads stand in for the pages' text, pixel-prediction and protein
sequence tasks ("Rethinking Attention with Performers", abstract): attention
speed does not depend on token identity, only on shape, and the value range
of the exponents is exercised by the offset workload.

Recipe (host generator): one numpy PCG64 stream ``default_rng(seed)``; for
each (b, h) in order: [offsets mu_Q, mu_K ~ N(0, 0.25 I_d) when enabled],
then Q, K, V rows via ``standard_normal(float32)``; Q and K are multiplied by
d^-1/4 and the offsets added; then the cast.  The device generator (for the
full-size timing and sampled-parity runs) follows the same recipe with a
seeded ``torch.Generator`` on the GPU, whole tensors at a time.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "host_qkv", "device_qkv"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    d: int
    m: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    offset_var: float   # variance of the per-head mean offset on Q and K (0 = none)
    seed_in: int
    seed_w: int
    redraw_every: int = 0   # calls between projection redraws (0 = never)

    @property
    def heads(self) -> int:
        return self.B * self.H

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _mk(c, **kw):
    return Workload(seed_in=1000 * c + 1, seed_w=1000 * c + 2, **kw)


# The five configurations: tiny fp32 check, text-length bidirectional and
# causal, protein-length with offsets, and the wide-head many-feature case.
WORKLOADS = {
    "tiny_f32": _mk(1, name="tiny_f32", B=1, H=1, L=256, d=16, m=16, dtype="f32",
                    causal=False, offset_var=0.0),
    "text_bidir": _mk(2, name="text_bidir", B=8, H=8, L=4096, d=64, m=256, dtype="bf16",
                      causal=False, offset_var=0.0),
    "text_causal": _mk(3, name="text_causal", B=8, H=8, L=4096, d=64, m=256, dtype="bf16",
                       causal=True, offset_var=0.0),
    "protein_long": _mk(4, name="protein_long", B=1, H=16, L=32768, d=64, m=256,
                        dtype="bf16", causal=False, offset_var=0.25),
    "wide_many": _mk(5, name="wide_many", B=4, H=32, L=16384, d=128, m=512, dtype="bf16",
                     causal=False, offset_var=0.0, redraw_every=10),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t if dtype == "f32" else t.to(torch.bfloat16)


def host_qkv(w: Workload, heads=None, L=None):
    """Q, K, V as CPU tensors [B, H, L, d] in the workload dtype.

    ``heads`` (an iterable of flat (b*H + h) indices) limits which heads are
    drawn; the stream still advances over every head before the last one
    requested, so a head's values do not depend on which others are drawn.
    ``L`` overrides the sequence length (the stream layout then changes).
    """
    L = w.L if L is None else L
    d = w.d
    rng = np.random.default_rng(w.seed_in)
    want = set(range(w.heads)) if heads is None else set(heads)
    last = max(want) if want else -1
    scale = np.float32(d ** -0.25)
    Q = np.zeros((w.heads, L, d), np.float32)
    K = np.zeros_like(Q)
    V = np.zeros_like(Q)
    for bh in range(last + 1):
        if w.offset_var > 0:
            muq = rng.standard_normal(d, dtype=np.float32) * np.float32(np.sqrt(w.offset_var))
            muk = rng.standard_normal(d, dtype=np.float32) * np.float32(np.sqrt(w.offset_var))
        else:
            muq = muk = np.zeros(d, np.float32)
        q = rng.standard_normal((L, d), dtype=np.float32)
        k = rng.standard_normal((L, d), dtype=np.float32)
        v = rng.standard_normal((L, d), dtype=np.float32)
        if bh in want:
            Q[bh] = q * scale + muq
            K[bh] = k * scale + muk
            V[bh] = v
    shp = (w.B, w.H, L, d)
    return (_cast(Q, w.dtype).reshape(shp), _cast(K, w.dtype).reshape(shp),
            _cast(V, w.dtype).reshape(shp))


def device_qkv(w: Workload, device="cuda", seed=None, L=None):
    """Q, K, V drawn directly on the device with a seeded torch generator."""
    L = w.L if L is None else L
    g = torch.Generator(device=device)
    g.manual_seed(w.seed_in if seed is None else seed)
    shp = (w.B, w.H, L, w.d)
    scale = w.d ** -0.25
    out = []
    for which in range(3):
        x = torch.randn(shp, generator=g, device=device, dtype=torch.float32)
        if which < 2:
            x.mul_(scale)
            if w.offset_var > 0:
                mu = torch.randn((w.B, w.H, 1, w.d), generator=g, device=device,
                                 dtype=torch.float32) * (w.offset_var ** 0.5)
                x.add_(mu)
        out.append(x.to(w.torch_dtype).contiguous())
    return tuple(out)
