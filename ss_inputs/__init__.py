"""Seeded synthetic inputs for the selective scan, shared by the tests, the
bench and the smoke check.

This module only draws random numbers and casts them; it holds none of the
scan's arithmetic.  Both the HIP path and the CPU oracle consume what it
returns, and neither imports the other.

Workloads (shapes are Mamba-1 layer widths; there is no dataset, the values
are drawn from the distributions below):

=========  ==  =======  ====  ==  ======  ======================================
name        B        L     D   N  io      optional tensors
=========  ==  =======  ====  ==  ======  ======================================
tiny        1      128    32  16  f32     none
m130m       4     1024  1536  16  f32     D skip, z, delta_bias, last_state
m2p8b       8     2048  5120  16  bf16    D skip, z, delta_bias (A/D/bias f32)
long        1   262144   512  16  f32     none
bwd         2     2048  2048  16  f32     D skip, z, delta_bias, dy
m2p8b_d8    8     2048   640  16  bf16    as m2p8b (one GPU's D / 8 share)
bwd_d8      2     2048   256  16  f32     as bwd (one GPU's D / 8 share)
=========  ==  =======  ====  ==  ======  ======================================

Distributions (numpy ``Generator(PCG64(seed))``, f64 draws in C order, drawn in
the order u, delta, B, C, z, Dskip, delta_bias, dy; absent tensors are not
drawn):

* ``u, B, C, z, dy ~ N(0, 1)``; ``delta ~ N(-1, 0.5)`` (pre-softplus);
* ``A[d, n] = -(n + 1)`` for every d (the S4D-real initialisation);
* ``Dskip ~ N(1, 0.1)``;
* ``delta_bias = log(expm1(s))`` with ``s`` log-uniform on ``[1e-3, 0.1]``,
  i.e. the bias whose softplus is ``s`` (the usual dt-bias initialisation).

Each tensor is then rounded once (round-to-nearest-even) to its storage dtype;
consumers read the rounded values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    dim: int
    dstate: int
    io_dtype: str = "f32"
    param_dtype: str = "f32"
    has_D: bool = False
    has_z: bool = False
    has_bias: bool = False
    last_state: bool = False
    backward: bool = False
    delta_softplus: bool = True
    seed: int = 0

    @property
    def updates(self) -> int:
        """Number of (b, t, d, n) state updates of one forward pass."""
        return self.batch * self.seqlen * self.dim * self.dstate

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 128, 32, 16, seed=1001),
    "m130m": Workload("m130m", 4, 1024, 1536, 16, has_D=True, has_z=True,
                      has_bias=True, last_state=True, seed=1002),
    "m2p8b": Workload("m2p8b", 8, 2048, 5120, 16, io_dtype="bf16",
                      param_dtype="f32", has_D=True, has_z=True,
                      has_bias=True, seed=1003),
    "long": Workload("long", 1, 262144, 512, 16, seed=1004),
    "bwd": Workload("bwd", 2, 2048, 2048, 16, has_D=True, has_z=True,
                    has_bias=True, backward=True, seed=1005),
    # one GPU's share of an 8-way split of the channels (D / 8): what a GPU of
    # an 8-GPU node runs for m2p8b and bwd, where the forward needs no
    # communication and the backward one sum of dB / dC
    "m2p8b_d8": Workload("m2p8b_d8", 8, 2048, 640, 16, io_dtype="bf16",
                         param_dtype="f32", has_D=True, has_z=True,
                         has_bias=True, seed=1006),
    "bwd_d8": Workload("bwd_d8", 2, 2048, 256, 16, has_D=True, has_z=True,
                       has_bias=True, backward=True, seed=1007),
}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))
    # torch's float64 -> {float32, float16, bfloat16} casts round to nearest even.
    return t.to(_TORCH_DTYPES[dtype]).contiguous()


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Draw the inputs of workload ``w`` as contiguous CPU tensors.

    Returns a dict with keys u, delta, A, B, C, D, z, delta_bias, dy (absent
    optional tensors map to None).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    Bn, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    io, pa = w.io_dtype, w.param_dtype
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["u"] = _cast(rng.normal(0.0, 1.0, size=(Bn, L, D)), io)
    out["delta"] = _cast(rng.normal(-1.0, 0.5, size=(Bn, L, D)), io)
    out["B"] = _cast(rng.normal(0.0, 1.0, size=(Bn, L, N)), io)
    out["C"] = _cast(rng.normal(0.0, 1.0, size=(Bn, L, N)), io)
    out["z"] = _cast(rng.normal(0.0, 1.0, size=(Bn, L, D)), io) if w.has_z else None
    out["D"] = _cast(rng.normal(1.0, 0.1, size=(D,)), pa) if w.has_D else None
    if w.has_bias:
        s = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=(D,)))
        out["delta_bias"] = _cast(np.log(np.expm1(s)), pa)
    else:
        out["delta_bias"] = None
    out["dy"] = _cast(rng.normal(0.0, 1.0, size=(Bn, L, D)), io) if w.backward else None
    A = -np.broadcast_to(np.arange(1, N + 1, dtype=np.float64), (D, N))
    out["A"] = _cast(A, pa)
    return out


def random_inputs(batch: int, seqlen: int, dim: int, dstate: int, *, seed: int,
                  io_dtype: str = "f32", param_dtype: str = "f32",
                  has_D: bool = True, has_z: bool = True, has_bias: bool = True,
                  backward: bool = False, a_scale: float = 1.0,
                  random_A: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of an arbitrary shape with the same value distributions.

    With ``random_A`` the state matrix is ``-exp(N(0, 1)) * a_scale`` per
    (d, n) instead of the S4D-real ramp, so that tests see distinct decays.
    """
    w = Workload("custom", batch, seqlen, dim, dstate, io_dtype=io_dtype,
                 param_dtype=param_dtype, has_D=has_D, has_z=has_z,
                 has_bias=has_bias, backward=backward, seed=seed)
    out = make_inputs(w)
    if random_A:
        rng = np.random.Generator(np.random.PCG64(seed + 7919))
        out["A"] = _cast(-np.exp(rng.normal(0.0, 1.0, size=(dim, dstate))) * a_scale,
                         param_dtype)
    return out
