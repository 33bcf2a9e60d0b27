"""Seeded synthetic inputs for the selective-scan workloads.

This module holds the input recipe only: shapes, dtypes, distributions and the
seeded draw order.  It computes nothing the scan itself computes; both the CPU
oracle (tests) and the GPU path (tests, bench) take their inputs from here.

Workloads (shapes follow the Mamba model ladder and the million-token DNA
setting described on the pages; the datasets they were measured on are not
used -- these synthetic draws stand in for them):

  0  tiny fp32 scan          B=1   D=16   N=4  L=64
  1  130M-shaped layer scan  B=8   D=1536 N=16 L=2048   bf16 in / fp32 state
  2  2.8B-shaped layer scan  B=4   D=5120 N=16 L=2048   bf16 in / fp32 state
  3  DNA-like long scan      B=1   D=256  N=16 L=2**20  fp32, u = P[token]
  4  2.8B-shaped decode      B=256 D=5120 N=16, 128 single-token steps, bf16

Common distributions: A[d,n] = -(n+1) (S4D-real, A_log = log(n+1));
dt_bias[d] = log(expm1(dt0)) with log(dt0) ~ U[log 1e-3, log 1e-1] (the
inverse softplus of a log-uniform step); raw delta ~ 0.1*N(0,1);
u, z, B, C ~ N(0,1); D = 1 (workload 0) else N(1, 0.1); softplus on.
Draws are made in fp32 by numpy PCG64 (seed = workload index unless given)
and rounded to bf16 (round-to-nearest-even, via torch on the CPU) where the
workload is bf16.  Draw order: dt_bias, D, u (workload 3: P, tokens), delta,
z, B, C.  Decode: dt_bias, D, state, then per step (own seed stream) u, delta,
z, B, C.

SSD (Mamba-2 form, scalar decay per head; ``ssd_inputs``): x [B, H*P, L], dt
[B, H, L], A [H], B, C [B, N, L], D [H*P], dt_bias [H], z [B, H*P, L].  The
benchmark shape is the 2.8B-shaped layer as 80 heads of 64 channels (B=4,
d_inner=5120, N=16, L=2048, bf16).  A_h = -U[1, 16]; dt_bias per head as
above; raw dt ~ 0.1*N(0,1); x, z, B, C ~ N(0,1); D ~ N(1, 0.1).  Draw order:
A, dt_bias, D, x, dt, z, B, C.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "scan_inputs", "random_scan_inputs", "decode_params",
           "decode_state", "decode_step_inputs", "to_dtype", "ssd_inputs", "SSD_LAYER"]


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int          # scan length (decode workloads: number of steps)
    dtype: str           # "f32" or "bf16" (u, delta, z, B, C, y)
    kind: str = "scan"   # "scan" or "decode"
    d_one: bool = False  # D == 1 exactly
    u_tokens: bool = False  # u = P[token_t, d]

    @property
    def elements(self) -> int:
        """B*L*D (scan) or B*D per step (decode)."""
        if self.kind == "decode":
            return self.batch * self.dim
        return self.batch * self.dim * self.seqlen


WORKLOADS = {
    0: Workload(0, "tiny-fp32 scan B=1 D=16 N=4 L=64", 1, 16, 4, 64, "f32", d_one=True),
    1: Workload(1, "130M-shaped layer scan B=8 D=1536 N=16 L=2048", 8, 1536, 16, 2048, "bf16"),
    2: Workload(2, "2.8B-shaped layer scan B=4 D=5120 N=16 L=2048", 4, 5120, 16, 2048, "bf16"),
    3: Workload(3, "DNA-like long scan B=1 D=256 N=16 L=2^20", 1, 256, 16, 1 << 20, "f32", u_tokens=True),
    4: Workload(4, "2.8B-shaped decode B=256 D=5120 N=16 x128 steps", 256, 5120, 16, 128, "bf16", kind="decode"),
}


def to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 numpy array -> contiguous CPU torch tensor of `dtype` (bf16 by RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()
    if dtype == "f32":
        return t.contiguous()
    raise ValueError(f"unknown dtype {dtype!r}")


def _rng(*seed) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))


def _normal(rng, shape, scale=1.0, mean=0.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _s4d_real_A(dim: int, dstate: int) -> torch.Tensor:
    # A_log[d, n] = log(n + 1)  =>  A = -exp(A_log) = -(n + 1), exact in fp32.
    a = -np.broadcast_to(np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate))
    return torch.from_numpy(np.ascontiguousarray(a))


def _dt_bias(rng, dim: int, dt_min=1e-3, dt_max=1e-1) -> torch.Tensor:
    # Inverse softplus of a log-uniform target step dt0:  log(exp(dt0) - 1).
    log_dt0 = rng.uniform(math.log(dt_min), math.log(dt_max), size=dim)
    dt0 = np.exp(log_dt0)
    return torch.from_numpy(np.log(np.expm1(dt0)).astype(np.float32))


def _D(rng, dim: int, one: bool) -> torch.Tensor:
    if one:
        return torch.ones(dim, dtype=torch.float32)
    return torch.from_numpy(_normal(rng, (dim,), 0.1, 1.0))


def scan_inputs(w: Workload | int, seed: int | None = None) -> dict:
    """Full-size inputs of scan workload `w` (CPU tensors)."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    assert w.kind == "scan"
    seed = w.index if seed is None else seed
    rng = _rng(seed)
    Bt, Dm, N, L = w.batch, w.dim, w.dstate, w.seqlen
    dt_bias = _dt_bias(rng, Dm)
    D = _D(rng, Dm, w.d_one)
    if w.u_tokens:
        P = _normal(rng, (4, Dm))
        tokens = rng.integers(0, 4, size=(Bt, L))
        u = np.empty((Bt, Dm, L), dtype=np.float32)
        for b in range(Bt):
            u[b] = P.T[:, tokens[b]]
    else:
        u = _normal(rng, (Bt, Dm, L))
    delta = _normal(rng, (Bt, Dm, L), 0.1)
    z = _normal(rng, (Bt, Dm, L))
    B = _normal(rng, (Bt, N, L))
    C = _normal(rng, (Bt, N, L))
    return dict(u=to_dtype(u, w.dtype), delta=to_dtype(delta, w.dtype), A=_s4d_real_A(Dm, N),
                B=to_dtype(B, w.dtype), C=to_dtype(C, w.dtype), D=D, z=to_dtype(z, w.dtype),
                dt_bias=dt_bias, softplus=True, batch=Bt, dim=Dm, dstate=N, seqlen=L, dtype=w.dtype)


def device_scan_inputs(batch: int, dim: int, dstate: int, seqlen: int, seed: int, device,
                       dtype: str = "bf16") -> dict:
    """Scan inputs too large to draw on the host, drawn on `device` (the workloads' distributions).

    u, z, B, C ~ N(0, 1), delta ~ 0.1 N(0, 1), from torch's seeded generator on that device, one batch row at a
    time in fp32 (rounded to bf16 for dtype "bf16"); A (S4D-real), dt_bias and D (N(1, 0.1)) from the host
    generator as for the workloads.  Both sides read the same device bytes: a checker copies back only the rows
    it samples.
    """
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = _rng(seed)
    dt_bias = _dt_bias(rng, dim)
    D = _D(rng, dim, False)
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def draw(rows, scale=1.0):
        out = torch.empty((batch, rows, seqlen), dtype=tdt, device=device)
        for b in range(batch):
            out[b] = (torch.randn((rows, seqlen), generator=g, device=device, dtype=torch.float32) * scale).to(tdt)
        return out

    u = draw(dim)
    delta = draw(dim, 0.1)
    z = draw(dim)
    B = draw(dstate)
    C = draw(dstate)
    return dict(u=u, delta=delta, A=_s4d_real_A(dim, dstate).to(device), B=B, C=C, D=D.to(device), z=z,
                dt_bias=dt_bias.to(device), softplus=True, batch=batch, dim=dim, dstate=dstate, seqlen=seqlen,
                dtype=dtype)


def random_scan_inputs(batch: int, dim: int, dstate: int, seqlen: int, dtype: str = "f32", seed: int = 0,
                       with_D: bool = True, with_z: bool = True, with_bias: bool = True,
                       softplus: bool = True, delta_scale: float = 0.1, a_mode: str = "s4d") -> dict:
    """Small random inputs with the workload distributions, for parity and property tests.

    a_mode: "s4d" -> A = -(n+1); "random" -> A = -exp(N(0,1)) per (d, n).
    """
    rng = _rng(10_000 + seed, batch, dim, dstate, seqlen)
    dt_bias = _dt_bias(rng, dim) if with_bias else None
    D = _D(rng, dim, False) if with_D else None
    u = _normal(rng, (batch, dim, seqlen))
    delta = _normal(rng, (batch, dim, seqlen), delta_scale)
    z = _normal(rng, (batch, dim, seqlen)) if with_z else None
    B = _normal(rng, (batch, dstate, seqlen))
    C = _normal(rng, (batch, dstate, seqlen))
    if a_mode == "s4d":
        A = _s4d_real_A(dim, dstate)
    else:
        A = torch.from_numpy(-np.exp(_normal(rng, (dim, dstate))))
    return dict(u=to_dtype(u, dtype), delta=to_dtype(delta, dtype), A=A, B=to_dtype(B, dtype),
                C=to_dtype(C, dtype), D=D, z=None if z is None else to_dtype(z, dtype), dt_bias=dt_bias,
                softplus=softplus, batch=batch, dim=dim, dstate=dstate, seqlen=seqlen, dtype=dtype)


def decode_params(w: Workload | int = 4, seed: int | None = None) -> dict:
    """Step-invariant decode inputs: A, D, dt_bias."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    seed = w.index if seed is None else seed
    rng = _rng(seed)
    dt_bias = _dt_bias(rng, w.dim)
    D = _D(rng, w.dim, w.d_one)
    return dict(A=_s4d_real_A(w.dim, w.dstate), D=D, dt_bias=dt_bias)


def decode_state(w: Workload | int = 4, seed: int | None = None) -> torch.Tensor:
    """Initial fp32 state [B, D, N] ~ N(0, 1)."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    seed = w.index if seed is None else seed
    rng = _rng(seed, 1)
    return torch.from_numpy(_normal(rng, (w.batch, w.dim, w.dstate)))


def decode_step_inputs(w: Workload | int, step: int, seed: int | None = None) -> dict:
    """Per-step decode inputs: u, delta, z [B, D] and B, C [B, N] (dtype of the workload)."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    seed = w.index if seed is None else seed
    rng = _rng(seed, 2, step)
    u = _normal(rng, (w.batch, w.dim))
    delta = _normal(rng, (w.batch, w.dim), 0.1)
    z = _normal(rng, (w.batch, w.dim))
    B = _normal(rng, (w.batch, w.dstate))
    C = _normal(rng, (w.batch, w.dstate))
    return dict(u=to_dtype(u, w.dtype), delta=to_dtype(delta, w.dtype), z=to_dtype(z, w.dtype),
                B=to_dtype(B, w.dtype), C=to_dtype(C, w.dtype))


SSD_LAYER = dict(batch=4, heads=80, headdim=64, dstate=16, seqlen=2048, dtype="bf16")


def ssd_inputs(batch: int, heads: int, headdim: int, dstate: int, seqlen: int, dtype: str = "bf16",
               seed: int = 0, with_D: bool = True, with_z: bool = True, with_bias: bool = True,
               softplus: bool = True) -> dict:
    """Inputs of the SSD (Mamba-2) layer: per-head scalar decay A [H], step dt [B, H, L]."""
    rng = _rng(20_000 + seed, batch, heads, headdim, dstate, seqlen)
    dim = heads * headdim
    A = torch.from_numpy(-rng.uniform(1.0, 16.0, size=heads).astype(np.float32))
    dt_bias = _dt_bias(rng, heads) if with_bias else None
    D = _D(rng, dim, False) if with_D else None
    x = _normal(rng, (batch, dim, seqlen))
    dt = _normal(rng, (batch, heads, seqlen), 0.1)
    z = _normal(rng, (batch, dim, seqlen)) if with_z else None
    B = _normal(rng, (batch, dstate, seqlen))
    C = _normal(rng, (batch, dstate, seqlen))
    return dict(x=to_dtype(x, dtype), dt=to_dtype(dt, dtype), A=A, B=to_dtype(B, dtype), C=to_dtype(C, dtype),
                D=D, z=None if z is None else to_dtype(z, dtype), dt_bias=dt_bias, softplus=softplus,
                batch=batch, heads=heads, headdim=headdim, dstate=dstate, seqlen=seqlen, dtype=dtype)
