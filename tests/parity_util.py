"""Shared helpers for the GPU parity tests (no method arithmetic here)."""
import sys

import numpy as np
import torch

KEYS = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")
GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias")

# Bounds from the target: max relative error 1e-5 for f32 I/O, 2e-2 for f16/bf16 I/O.
TOL = {torch.float32: 1e-5, torch.float16: 2e-2, torch.bfloat16: 2e-2}


def rel_err(x, r) -> float:
    """max_i |x_i - r_i| / max(|r_i|, rms(r)).

    Plain elementwise relative error is ill-posed where outputs cancel to
    about 0 (a y is a random-sign sum), so each element is scaled by the
    larger of its own magnitude and the tensor's RMS.
    """
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        return float(np.max(np.abs(x - r)))
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms)))


def to_np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def to_dev(inp, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}


def say(*a):
    """Name the case before each GPU step (flushed, so it survives a crash)."""
    print(*a, flush=True)
    sys.stdout.flush()
