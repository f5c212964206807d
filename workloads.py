"""Seeded synthetic inputs for the selective scan (shared by tests and bench).

This module holds only sampling and storage rounding: none of the scan's
arithmetic.  Both the GPU path and the oracle read the arrays it returns.

Recipe (stated once here, repeated in the design doc):

* numpy ``PCG64``; every array gets its own child ``SeedSequence`` spawned from
  the workload seed in a fixed draw order (x, z, B, C, step-size draw,
  per-channel step-size draw, D).  Large arrays are filled in fixed 4 Mi-element
  chunks, each from its own grandchild seed, so the values do not depend on the
  number of threads used.
* Samples are drawn in float32 and rounded once to the storage dtype
  (round-to-nearest-even); for bf16 the arrays returned are float32 arrays
  whose values are exactly representable in bf16.
* ``A[d, n] = -(n + 1)`` (the S4D-Real initialisation of the page-3 report,
  section 3 "MambaBlock"), ``D ~ N(0, 1)`` per channel.
* Step sizes: for the "log-uniform" workloads a per-channel bias is placed at
  ``bias[d] = softplus^-1(Delta0[d])`` and ``dt = softplus^-1(Delta*) - bias[d]``
  with ``Delta0, Delta* ~ logU[lo, hi]``, so the step size seen by the method is
  ``Delta*`` up to the rounding of ``dt`` and the bias path is exercised.  (The
  inverse ``softplus^-1(u) = log(expm1(u))`` only places the inputs.)
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to the nearest bfloat16 (ties to even); returns float32."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(dtype)


def _chunked(ss: np.random.SeedSequence, shape, fill) -> np.ndarray:
    """Fill a float32 array of ``shape`` chunk by chunk; ``fill(rng, out)`` writes one chunk."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + CHUNK - 1) // CHUNK)
    kids = ss.spawn(nchunks)

    def work(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        if hi > lo:
            fill(np.random.Generator(np.random.PCG64(kids[i])), out[lo:hi])

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def _normal(ss, shape, scale=1.0):
    def fill(rng, o):
        rng.standard_normal(out=o, dtype=np.float32)
        if scale != 1.0:
            o *= np.float32(scale)
    return _chunked(ss, shape, fill)


def _uniform(ss, shape, lo, hi):
    def fill(rng, o):
        rng.random(out=o, dtype=np.float32)
        o *= np.float32(hi - lo)
        o += np.float32(lo)
    return _chunked(ss, shape, fill)


def _inv_softplus(u: np.ndarray) -> np.ndarray:
    u = np.asarray(u, dtype=np.float64)
    return np.log(np.expm1(u))


def _dt_logu(ss, shape, bias: np.ndarray, lo: float, hi: float) -> np.ndarray:
    """dt = softplus^-1(Delta*) - bias[d], Delta* ~ logU[lo, hi] (float32 result, unrounded)."""
    llo, lhi = np.log(lo), np.log(hi)
    b64 = bias.astype(np.float64)
    dim = shape[-1]

    def fill(rng, o):
        # chunks are whole multiples of dim whenever dim divides CHUNK; handle the general case
        u = rng.random(o.shape[0], dtype=np.float64)
        dstar = np.exp(llo + (lhi - llo) * u)
        o[:] = _inv_softplus(dstar)
    flat = _chunked(ss, shape, fill).reshape(-1, dim)
    flat -= b64.astype(np.float32)[None, :]
    return flat.reshape(shape)


@dataclass
class ScanInputs:
    """Inputs of one forward scan.  Arrays are float32; for dtype "bf16" the values of
    x, dt, z, B, C are exactly representable in bfloat16.  A, D, dt_bias are fp32."""
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    dtype: str
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: Optional[np.ndarray]
    z: Optional[np.ndarray]
    dt_bias: Optional[np.ndarray]
    meta: Dict = field(default_factory=dict)


def s4d_real_A(dim: int, dstate: int) -> np.ndarray:
    """A[d, n] = -(n + 1), float32."""
    return np.ascontiguousarray(-np.broadcast_to(np.arange(1, dstate + 1, dtype=np.float32), (dim, dstate)))


def make_scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, dtype: str = "f32",
                     seed: int = 0, step: str = "logu", delta_range: Tuple[float, float] = (1e-3, 1e-1),
                     dt_uniform: Tuple[float, float] = (-4.0, -2.0), with_z: bool = True,
                     with_D: bool = True, with_bias: bool = True, name: str = "custom") -> ScanInputs:
    """General seeded workload.

    step == "logu":    Delta ~ logU[delta_range] through a per-channel bias (see module doc).
    step == "uniform": dt ~ U(dt_uniform), bias = zeros if with_bias else absent.
    step == "normal":  dt ~ N(0, 1), bias absent.
    """
    kids = np.random.SeedSequence(seed).spawn(8)
    shp3 = (batch, seqlen, dim)
    shpn = (batch, seqlen, dstate)
    x = _normal(kids[0], shp3)
    z = _normal(kids[1], shp3) if with_z else None
    B = _normal(kids[2], shpn)
    C = _normal(kids[3], shpn)
    bias = None
    if step == "logu":
        lo, hi = delta_range
        d0 = np.exp(np.log(lo) + (np.log(hi) - np.log(lo)) *
                    np.random.Generator(np.random.PCG64(kids[5])).random(dim))
        bias = _inv_softplus(d0).astype(np.float32)
        dt = _dt_logu(kids[4], shp3, bias, lo, hi)
        if not with_bias:
            dt = dt + bias[None, None, :]
            bias = None
    elif step == "uniform":
        dt = _uniform(kids[4], shp3, dt_uniform[0], dt_uniform[1])
        bias = np.zeros(dim, dtype=np.float32) if with_bias else None
    elif step == "normal":
        dt = _normal(kids[4], shp3)
    else:
        raise ValueError(step)
    D = _normal(kids[6], (dim,)) if with_D else None
    return ScanInputs(name=name, batch=batch, seqlen=seqlen, dim=dim, dstate=dstate, dtype=dtype,
                      x=_store(x, dtype), dt=_store(dt, dtype), A=s4d_real_A(dim, dstate),
                      B=_store(B, dtype), C=_store(C, dtype), D=D, z=None if z is None else _store(z, dtype),
                      dt_bias=bias, meta=dict(seed=seed, step=step, delta_range=delta_range))


def device_scan_inputs(batch: int, seqlen: int, dim: int, dstate: int, seed: int,
                       delta_range: Tuple[float, float] = (1e-3, 1e-1), device: str = "cuda") -> Dict:
    """Seeded bf16 inputs drawn on the device, for shapes whose tensors are too large
    to sample on the host (several GB each).  The recipe of make_scan_inputs with
    step == "logu" (x, z, B, C ~ N(0, 1); per-channel bias = softplus^-1(Delta0),
    dt = softplus^-1(Delta*) - bias with Delta0, Delta* ~ logU[delta_range];
    A = -(n + 1); D ~ N(0, 1)), drawn with torch's device generator seeded by `seed`,
    one batch row at a time, in float32 and rounded once to bf16.  Also an upstream
    gradient dy ~ N(0, 1) (bf16) and dlast ~ N(0, 1) (float32) for the backward pass.
    Returns a dict of device tensors: x, dt, z, dy, B, C (bf16); A, D, dt_bias, dlast
    (float32)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    f32, bf = torch.float32, torch.bfloat16
    llo, lhi = float(np.log(delta_range[0])), float(np.log(delta_range[1]))

    def logu(shape):
        return torch.exp(llo + (lhi - llo) * torch.rand(shape, generator=gen, device=device, dtype=f32))

    d0 = logu((dim,))
    bias = torch.log(torch.expm1(d0))
    out = {name: torch.empty((batch, seqlen, dim), dtype=bf, device=device) for name in ("x", "dt", "z", "dy")}
    for b in range(batch):
        out["x"][b] = torch.randn((seqlen, dim), generator=gen, device=device, dtype=f32).to(bf)
        out["z"][b] = torch.randn((seqlen, dim), generator=gen, device=device, dtype=f32).to(bf)
        out["dt"][b] = (torch.log(torch.expm1(logu((seqlen, dim)))) - bias[None, :]).to(bf)
        out["dy"][b] = torch.randn((seqlen, dim), generator=gen, device=device, dtype=f32).to(bf)
    out["B"] = torch.randn((batch, seqlen, dstate), generator=gen, device=device, dtype=f32).to(bf)
    out["C"] = torch.randn((batch, seqlen, dstate), generator=gen, device=device, dtype=f32).to(bf)
    out["A"] = torch.from_numpy(s4d_real_A(dim, dstate)).to(device)
    out["D"] = torch.randn((dim,), generator=gen, device=device, dtype=f32)
    out["dt_bias"] = bias
    out["dlast"] = torch.randn((batch, dim, dstate), generator=gen, device=device, dtype=f32)
    return out


def device_step_inputs(batch: int, dim: int, dstate: int, seed: int, device: str = "cuda") -> Dict:
    """Seeded inputs of one decode step drawn on the device, for states too large to
    sample on the host: the recipe of DecodeWorkload (state ~ 0.1 N(0, 1) float32;
    x, dt, z [batch, dim] and B, C [batch, dstate] ~ N(0, 1) in bf16; A = -(n + 1);
    D ~ N(0, 1); no bias), drawn with torch's device generator seeded by `seed`."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    f32, bf = torch.float32, torch.bfloat16
    state = torch.empty((batch, dim, dstate), dtype=f32, device=device)
    for b in range(batch):
        state[b] = 0.1 * torch.randn((dim, dstate), generator=gen, device=device, dtype=f32)
    out = {"state": state}
    for name, shape in (("x", (batch, dim)), ("dt", (batch, dim)), ("z", (batch, dim)), ("B", (batch, dstate)),
                        ("C", (batch, dstate))):
        out[name] = torch.randn(shape, generator=gen, device=device, dtype=f32).to(bf)
    out["A"] = torch.from_numpy(s4d_real_A(dim, dstate)).to(device)
    out["D"] = torch.randn((dim,), generator=gen, device=device, dtype=f32)
    return out


# ----------------------------------------------------------------------------
# The five named workloads.
# ----------------------------------------------------------------------------
FWD_WORKLOADS = {
    # Tiny fwd scan: batch 1, L 64, D 16, N 4, fp32, dt ~ U(-4,-2), bias 0.
    "tiny": dict(batch=1, seqlen=64, dim=16, dstate=4, dtype="f32", seed=1, step="uniform",
                 dt_uniform=(-4.0, -2.0)),
    # Mamba-130m-like layer: batch 2, L 2048, D 1536, N 16, fp32, Delta ~ logU[1e-3, 1e-1].
    "mamba130m_layer": dict(batch=2, seqlen=2048, dim=1536, dstate=16, dtype="f32", seed=2,
                            step="logu", delta_range=(1e-3, 1e-1)),
    # Training shape: batch 8, L 4096, D 2048, N 16, bf16 inputs, fp32 A/D/state.
    "train_shape": dict(batch=8, seqlen=4096, dim=2048, dstate=16, dtype="bf16", seed=3,
                        step="logu", delta_range=(1e-3, 1e-1)),
    # Long context: batch 1, L 131072, D 2560, N 16, bf16, Delta ~ logU[1e-4, 1e-2].
    "long_context": dict(batch=1, seqlen=131072, dim=2560, dstate=16, dtype="bf16", seed=4,
                         step="logu", delta_range=(1e-4, 1e-2)),
}

# Recurrent decode: batch 256, D 5120, N 16, fp32 state ~ 0.1 N(0,1); bf16 tokens ~ N(0,1).
DECODE = dict(batch=256, dim=5120, dstate=16, dtype="bf16", seed=5, steps=1000)


def workload(name: str, **overrides) -> ScanInputs:
    cfg = dict(FWD_WORKLOADS[name])
    cfg.update(overrides)
    return make_scan_inputs(name=name, **cfg)


@dataclass
class DecodeToken:
    x: np.ndarray
    dt: np.ndarray
    z: np.ndarray
    B: np.ndarray
    C: np.ndarray


class DecodeWorkload:
    """Recurrent decode workload: a resident state and a stream of single tokens."""

    def __init__(self, batch=DECODE["batch"], dim=DECODE["dim"], dstate=DECODE["dstate"],
                 dtype=DECODE["dtype"], seed=DECODE["seed"]):
        self.batch, self.dim, self.dstate, self.dtype, self.seed = batch, dim, dstate, dtype, seed
        root = np.random.SeedSequence(seed)
        k_state, k_param, self._k_tokens = root.spawn(3)
        kp = k_param.spawn(2)
        self.state0 = _normal(k_state, (batch, dim, dstate), scale=0.1)
        self.A = s4d_real_A(dim, dstate)
        self.D = _normal(kp[0], (dim,))
        self.dt_bias = None

    def token(self, step: int) -> DecodeToken:
        """Token ``step`` (0-based): x, dt, z [batch, dim]; B, C [batch, dstate], all ~ N(0, 1)."""
        ss = np.random.SeedSequence([self.seed, 1 + step])
        kids = ss.spawn(5)
        bd, bn = (self.batch, self.dim), (self.batch, self.dstate)
        return DecodeToken(x=_store(_normal(kids[0], bd), self.dtype), dt=_store(_normal(kids[1], bd), self.dtype),
                           z=_store(_normal(kids[2], bd), self.dtype), B=_store(_normal(kids[3], bn), self.dtype),
                           C=_store(_normal(kids[4], bn), self.dtype))


def fwd_algorithmic_bytes(batch, seqlen, dim, dstate, dtype, with_z=True, with_D=True,
                          with_bias=True, with_state=True) -> int:
    """Bytes the forward scan must move: inputs read once, outputs written once."""
    s = 2 if dtype == "bf16" else 4
    tok = batch * seqlen * dim * (s * (3 if with_z else 2) + s)      # x, dt, (z) read; y written
    bc = 2 * batch * seqlen * dstate * s                               # B, C
    par = 4 * dim * dstate + 4 * dim * (int(with_D) + int(with_bias))  # A, D, bias
    st = 4 * batch * dim * dstate if with_state else 0                 # last_state written
    return tok + bc + par + st


def bwd_algorithmic_bytes(batch: int, seqlen: int, dim: int, dstate: int, dtype: str,
                          with_z: bool = True, with_D: bool = True, with_bias: bool = True) -> int:
    """Bytes the backward pass must move: x, dt, (z), dy read and dx, ddt, (dz) written
    once per (b, l, d); B, C read and dB, dC written once per (b, l, n); A, (D), (bias)
    read and their gradients written once.  Checkpoints and partial sums are not
    counted (they are the implementation's choice, not the method's)."""
    s = 2 if dtype == "bf16" else 4
    tok = batch * seqlen * dim * s * ((4 if with_z else 3) + (3 if with_z else 2))
    bc = batch * seqlen * dstate * s * 4
    par = 4 * dim * dstate * 2 + 4 * dim * ((2 if with_D else 0) + (2 if with_bias else 0))
    return tok + bc + par


def step_algorithmic_bytes(batch, dim, dstate, dtype, with_z=True, with_D=True, with_bias=False) -> int:
    """Bytes one decode step must move: state read + written, token tensors, parameters."""
    s = 2 if dtype == "bf16" else 4
    return (8 * batch * dim * dstate + batch * dim * (s * (3 if with_z else 2) + s)
            + 2 * batch * dstate * s + 4 * dim * dstate + 4 * dim * (int(with_D) + int(with_bias)))
