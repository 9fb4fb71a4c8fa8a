"""Seeded synthetic inputs drawn on the GPU, for cases too large to draw on the host and ship
over (tensors past 2^31 elements).

Same recipe as ``make_inputs``: x, z ~ N(0,1); dt_raw ~ 0.5*N(0,1); B, C ~ N(0,1); dy, h0 ~
N(0,1), narrowed to bfloat16 by torch's round-to-nearest-even cast for bf16 cases.  Each big
tensor has its own torch device generator, seeded from the case seed and the tensor's index
in ``STREAMS``; the per-channel parameters (dt_bias, A, Dskip) come from the same numpy
streams as ``make_inputs`` with that seed, so they equal a host draw of the same case.
``channel(b, d)`` copies one channel's rows back as a (B=1, D=1) host case for the oracle:
the exact values the GPU read.  This module holds none of the scan's arithmetic.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .inputs import STREAMS, S6Inputs, make_inputs


def _device_normal(shape, seed, stream, scale, dtype, device):
    """A seeded N(0, scale^2) tensor of `shape` in `dtype`, drawn one slab of the first
    dimension at a time (bounds the float32 temporary)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 64 + STREAMS.index(stream))
    out = torch.empty(shape, dtype=dtype, device=device)
    for i in range(shape[0]):
        v = torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            v.mul_(scale)
        out[i].copy_(v)
        del v
    return out


@dataclass
class DeviceCase:
    """A case whose sequence tensors live on the GPU (torch tensors, order 0: [B, D, L] and
    [B, N, L]; order 1: [B, L, D] and [B, L, N]); per-channel parameters on both sides."""
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str
    order: int
    x: object
    dt_raw: object
    Bm: object
    Cm: object
    z: Optional[object]
    dy: Optional[object]
    h0: Optional[object]
    dt_bias: np.ndarray
    A: np.ndarray
    Dskip: np.ndarray
    dt_bias_t: object = None
    A_t: object = None
    Dskip_t: object = None

    def _row(self, t, b, d):
        """Channel (b, d) of a [B, D, L] (order 0) or [B, L, D] (order 1) tensor, float32."""
        v = t[b, d, :] if self.order == 0 else t[b, :, d]
        return v.float().cpu().numpy()

    def _bc(self, t, b):
        """Batch row b of a [B, N, L] (order 0) or [B, L, N] (order 1) tensor as [N, L]."""
        v = t[b] if self.order == 0 else t[b].t()
        return np.ascontiguousarray(v.float().cpu().numpy())

    def channel(self, b: int, d: int) -> S6Inputs:
        """Channel (b, d) as a one-channel host case (arrays shaped B = 1, D = 1)."""
        L, N = self.seqlen, self.dstate
        row = lambda t: None if t is None else self._row(t, b, d).reshape(1, 1, L)
        h0 = None if self.h0 is None else self.h0[b, d].float().cpu().numpy().reshape(1, 1, N)
        return S6Inputs(1, L, 1, N, self.dtype, row(self.x), row(self.dt_raw),
                        self.dt_bias[d:d + 1].copy(), self.A[d:d + 1].copy(),
                        self._bc(self.Bm, b).reshape(1, N, L), self._bc(self.Cm, b).reshape(1, N, L),
                        self.Dskip[d:d + 1].copy(), z=row(self.z), h0=h0, dy=row(self.dy),
                        meta=dict(b=b, d=d))


def make_device_inputs(batch: int, seqlen: int, dim: int, dstate: int, *, dtype: str = "bf16",
                       seed: int = 0, gate: bool = True, a_perturb: bool = True, order: int = 0,
                       with_dy: bool = False, with_h0: bool = False,
                       device: str = "cuda") -> DeviceCase:
    import torch
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"dtype must be 'f32' or 'bf16', got {dtype!r}")
    Bn, L, D, N = batch, seqlen, dim, dstate
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    seq = (Bn, D, L) if order == 0 else (Bn, L, D)
    bcs = (Bn, N, L) if order == 0 else (Bn, L, N)
    x = _device_normal(seq, seed, "x", 1.0, tdt, device)
    dt_raw = _device_normal(seq, seed, "dt_raw", 0.5, tdt, device)
    z = _device_normal(seq, seed, "z", 1.0, tdt, device) if gate else None
    Bm = _device_normal(bcs, seed, "B", 1.0, tdt, device)
    Cm = _device_normal(bcs, seed, "C", 1.0, tdt, device)
    dy = _device_normal(seq, seed, "dy", 1.0, torch.float32, device) if with_dy else None
    h0 = _device_normal((Bn, D, N), seed, "h0", 1.0, torch.float32, device) if with_h0 else None
    # per-channel parameters: the host draw of make_inputs (independent streams)
    p = make_inputs(1, 1, D, N, seed=seed, a_perturb=a_perturb)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    return DeviceCase(Bn, L, D, N, dtype, order, x, dt_raw, Bm, Cm, z, dy, h0,
                      p.dt_bias, p.A, p.Dskip, f32(p.dt_bias), f32(p.A), f32(p.Dskip))
