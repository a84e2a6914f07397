"""CPU oracle for the Mamba-1 selective scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg may import this package.  It shares no code with the
HIP library and never imports it.

Two independent implementations of the same definition:

* ``fwd`` / ``bwd`` / ``fwd_channels``: ctypes wrappers around the C loop in
  ``ss_oracle.c`` (double precision, threaded over channels).  ``fwd_f32`` /
  ``bwd_f32`` run the same loop in float (the single-precision rounding floor).
* ``np_fwd`` / ``np_bwd``: a numpy implementation, vectorised over the (b, d)
  channels and looping over time, used to cross-check the C code on small
  shapes.

What is computed (baracuda-kernels page "src/attention/selective_scan.rs",
module docs, "Algorithm summary" and "Shape contract"; gradient set from that
page's SelectiveScanBackwardArgs; backward equations derived by the chain
rule, the per-channel reverse sweep following stage B3 "SSM BPTT +
reductions" of the mamba-rs page "mamba_ssm/gpu/backward.rs"):

    x  = delta[b,t,d] + delta_bias[d]               (bias optional)
    dt = softplus(x) if delta_softplus else x
    a  = exp(dt * A[d,n])
    h  = a * h + dt * B[b,t,n] * u[b,t,d]           (h = h0 or 0 before t = 0)
    o  = sum_n C[b,t,n] * h[n] + D[d] * u[b,t,d]    (D optional)
    y  = o * z * sigmoid(z)                          (z optional)

The optional initial state h0 [B, D, N] is the per-layer SSM state that the
forward pipeline of the mamba-rs page "mamba_ssm/gpu/backward.rs" carries from
one call to the next; its gradient dh0 = dL/dh_{-1} is what the reverse sweep
carries past t = 0.

Packed variable-length sequences (``fwd_varlen`` / ``bwd_varlen``; the scan
page leaves cu_seqlens out of its scope, "Trailblazer scope") are read the
usual way: each sequence is an independent scan of its rows.

Inputs are decoded to float64 from whatever dtype they are stored in, so the
oracle reads exactly the values the GPU reads.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SS_ORACLE_LIB lets the mutation test point the wrapper at a deliberately
# broken build of the same source.
_LIB_PATH = os.environ.get("SS_ORACLE_LIB") or os.path.join(_HERE, "libss_oracle.so")
_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("dim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("delta_softplus", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        vp = ctypes.c_void_p
        for name in ("ss_oracle_fwd_f64", "ss_oracle_fwd_f32"):
            f = getattr(lib, name)
            f.argtypes = [ctypes.POINTER(_Problem)] + [vp] * 11 + [ctypes.c_int]
            f.restype = ctypes.c_int
        f = lib.ss_oracle_fwd_channels_f64
        f.argtypes = [ctypes.POINTER(_Problem)] + [vp] * 11 + [ctypes.c_int64, vp, vp,
                                                                ctypes.c_int]
        f.restype = ctypes.c_int
        for name in ("ss_oracle_bwd_f64", "ss_oracle_bwd_f32"):
            f = getattr(lib, name)
            f.argtypes = [ctypes.POINTER(_Problem)] + [vp] * 19 + [ctypes.c_int]
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _arr(x, dt) -> Optional[np.ndarray]:
    """Decode a torch tensor / numpy array / sequence to a contiguous array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: decode its stored values exactly
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64), dtype=dt)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _shape(u, A, delta_softplus) -> _Problem:
    Bn, L, D = u.shape
    N = A.shape[1]
    return _Problem(Bn, L, D, N, 1 if delta_softplus else 0)


def _check_shapes(u, delta, A, B, C, D, z, bias, dy=None, h0=None):
    Bn, L, Dd = u.shape
    N = A.shape[1]
    assert h0 is None or h0.shape == (Bn, Dd, N)
    assert delta.shape == (Bn, L, Dd) and A.shape == (Dd, N)
    assert B.shape == (Bn, L, N) and C.shape == (Bn, L, N)
    assert D is None or D.shape == (Dd,)
    assert z is None or z.shape == (Bn, L, Dd)
    assert bias is None or bias.shape == (Dd,)
    assert dy is None or dy.shape == (Bn, L, Dd)


def _fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
         return_last_state=False, nthreads=None, dt=np.float64, h0=None):
    args = [_arr(t, dt) for t in (u, delta, A, B, C, D, z, delta_bias)]
    h0a = _arr(h0, dt)
    _check_shapes(*args, h0=h0a)
    p = _shape(args[0], args[2], delta_softplus)
    y = np.empty(args[0].shape, dtype=dt)
    ls = np.empty((p.batch, p.dim, p.dstate), dtype=dt) if return_last_state else None
    fn = _load().ss_oracle_fwd_f64 if dt == np.float64 else _load().ss_oracle_fwd_f32
    st = fn(ctypes.byref(p), *[_ptr(a) for a in args], _ptr(h0a), _ptr(y), _ptr(ls),
            nthreads or default_threads())
    if st != 0:
        raise RuntimeError("oracle forward failed")
    return y, ls


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
        return_last_state=False, nthreads=None, h0=None):
    """Forward in float64.  Returns (y [B,L,D], last_state [B,D,N] or None).
    h0 [B,D,N]: state before t = 0 (zero when None)."""
    return _fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, return_last_state,
                nthreads, np.float64, h0)


def fwd_f32(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
            return_last_state=False, nthreads=None, h0=None):
    """The same sequential loop in float32 (diagnostic rounding floor)."""
    return _fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, return_last_state,
                nthreads, np.float32, h0)


def fwd_channels(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 chan_b: Sequence[int] = (), chan_d: Sequence[int] = (), nthreads=None,
                 h0=None):
    """Forward of selected channels only.

    Returns (y [nchan, L], last_state [nchan, N]) for channels
    (chan_b[c], chan_d[c]).
    """
    args = [_arr(t, np.float64) for t in (u, delta, A, B, C, D, z, delta_bias)]
    h0a = _arr(h0, np.float64)
    _check_shapes(*args, h0=h0a)
    p = _shape(args[0], args[2], delta_softplus)
    cb = np.ascontiguousarray(chan_b, dtype=np.int64)
    cd = np.ascontiguousarray(chan_d, dtype=np.int64)
    assert cb.shape == cd.shape and cb.ndim == 1
    y = np.empty((cb.size, p.seqlen), dtype=np.float64)
    ls = np.empty((cb.size, p.dstate), dtype=np.float64)
    st = _load().ss_oracle_fwd_channels_f64(ctypes.byref(p), *[_ptr(a) for a in args],
                                            _ptr(h0a), _ptr(cb), _ptr(cd), cb.size, _ptr(y),
                                            _ptr(ls),
                                            nthreads or default_threads())
    if st != 0:
        raise RuntimeError("oracle channel forward failed")
    return y, ls


def _bwd(u, delta, A, B, C, D, z, delta_bias, dy, delta_softplus, nthreads, dt, h0=None):
    args = [_arr(t, dt) for t in (u, delta, A, B, C, D, z, delta_bias)]
    h0a = _arr(h0, dt)
    dya = _arr(dy, dt)
    _check_shapes(*args, dy=dya, h0=h0a)
    p = _shape(args[0], args[2], delta_softplus)
    Bn, L, Dd, N = p.batch, p.seqlen, p.dim, p.dstate
    out = {
        "du": np.empty((Bn, L, Dd), dt), "ddelta": np.empty((Bn, L, Dd), dt),
        "dA": np.empty((Dd, N), dt), "dB": np.empty((Bn, L, N), dt),
        "dC": np.empty((Bn, L, N), dt),
        "dD": np.empty((Dd,), dt) if args[5] is not None else None,
        "dz": np.empty((Bn, L, Dd), dt) if args[6] is not None else None,
        "ddelta_bias": np.empty((Dd,), dt) if args[7] is not None else None,
        "dh0": np.empty((Bn, Dd, N), dt) if h0a is not None else None,
    }
    fn = _load().ss_oracle_bwd_f64 if dt == np.float64 else _load().ss_oracle_bwd_f32
    st = fn(ctypes.byref(p), *[_ptr(a) for a in args], _ptr(h0a), _ptr(dya),
            *[_ptr(out[k]) for k in ("du", "ddelta", "dA", "dB", "dC", "dD", "dz",
                                     "ddelta_bias", "dh0")],
            nthreads or default_threads())
    if st != 0:
        raise RuntimeError("oracle backward failed")
    return out


def bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None, delta_softplus=True,
        nthreads=None, h0=None) -> Dict[str, Optional[np.ndarray]]:
    """Backward in float64: gradients of sum(dy * y) with respect to every input.

    Returns a dict with du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0 (the
    last four are None when D / z / delta_bias / h0 are absent).
    """
    return _bwd(u, delta, A, B, C, D, z, delta_bias, dy, delta_softplus, nthreads, np.float64,
                h0)


def bwd_f32(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None, delta_softplus=True,
            nthreads=None, h0=None) -> Dict[str, Optional[np.ndarray]]:
    return _bwd(u, delta, A, B, C, D, z, delta_bias, dy, delta_softplus, nthreads, np.float32,
                h0)


# --------------------------------------------------------------------------
# Packed variable-length sequences: each sequence is its own scan.
# --------------------------------------------------------------------------

def _segments(cu_seqlens):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert cu.ndim == 1 and cu[0] == 0 and np.all(np.diff(cu) >= 0)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(cu.size - 1)]


def _seg(x, a, b):
    """Rows a..b of a packed [T, C] tensor as a [1, b - a, C] batch."""
    return None if x is None else _arr(x, np.float64)[a:b][None]


def fwd_varlen(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
               cu_seqlens=(0,), h0=None, nthreads=None):
    """Forward over packed sequences: u, delta, z [T, D]; B, C [T, N];
    sequence s is rows cu_seqlens[s] .. cu_seqlens[s+1] - 1, scanned from
    h0[s] (or 0).  Returns (y [T, D], last_state [S, D, N])."""
    segs = _segments(cu_seqlens)
    Dd, N = _arr(A, np.float64).shape
    y = np.zeros(_arr(u, np.float64).shape)
    ls = np.zeros((len(segs), Dd, N))
    h0a = _arr(h0, np.float64)
    for s, (a, b) in enumerate(segs):
        ys, lss = fwd(_seg(u, a, b), _seg(delta, a, b), A, _seg(B, a, b), _seg(C, a, b), D,
                      _seg(z, a, b), delta_bias, delta_softplus, return_last_state=True,
                      nthreads=nthreads, h0=None if h0a is None else h0a[s:s + 1])
        y[a:b] = ys[0]
        ls[s] = lss[0]
    return y, ls


def bwd_varlen(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None,
               delta_softplus=True, cu_seqlens=(0,), h0=None, nthreads=None):
    """Backward of ``fwd_varlen`` for the loss sum(dy * y): per-row gradients
    in the packed layout, parameter gradients summed over the sequences in
    sequence order, dh0 [S, D, N] when h0 is given."""
    segs = _segments(cu_seqlens)
    Dd, N = _arr(A, np.float64).shape
    T = _arr(u, np.float64).shape[0]
    h0a = _arr(h0, np.float64)
    out = {"du": np.zeros((T, Dd)), "ddelta": np.zeros((T, Dd)), "dA": np.zeros((Dd, N)),
           "dB": np.zeros((T, N)), "dC": np.zeros((T, N)),
           "dD": np.zeros(Dd) if D is not None else None,
           "dz": np.zeros((T, Dd)) if z is not None else None,
           "ddelta_bias": np.zeros(Dd) if delta_bias is not None else None,
           "dh0": np.zeros((len(segs), Dd, N)) if h0a is not None else None}
    for s, (a, b) in enumerate(segs):
        if b == a:
            continue
        g = bwd(_seg(u, a, b), _seg(delta, a, b), A, _seg(B, a, b), _seg(C, a, b), D,
                _seg(z, a, b), delta_bias, _seg(dy, a, b), delta_softplus, nthreads=nthreads,
                h0=None if h0a is None else h0a[s:s + 1])
        for k in ("du", "ddelta", "dB", "dC", "dz"):
            if out[k] is not None:
                out[k][a:b] = g[k][0]
        for k in ("dA", "dD", "ddelta_bias"):
            if out[k] is not None:
                out[k] += g[k]
        if h0a is not None:
            out["dh0"][s] = g["dh0"][0]
    return out


# --------------------------------------------------------------------------
# Independent numpy implementation (vectorised over channels, loop over t).
# --------------------------------------------------------------------------

def _np_softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _np_sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _np_prep(u, delta, A, B, C, D, z, delta_bias, delta_softplus):
    u, delta, A, B, C, D, z, bias = [_arr(t, np.float64)
                                     for t in (u, delta, A, B, C, D, z, delta_bias)]
    x = delta + (bias[None, None, :] if bias is not None else 0.0)
    dt = _np_softplus(x) if delta_softplus else x
    return u, A, B, C, D, z, x, dt


def np_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True, h0=None):
    """numpy forward (float64). Returns (y, last_state)."""
    u, A, B, C, D, z, x, dt = _np_prep(u, delta, A, B, C, D, z, delta_bias, delta_softplus)
    Bn, L, Dd = u.shape
    N = A.shape[1]
    h = np.zeros((Bn, Dd, N)) if h0 is None else _arr(h0, np.float64).copy()
    y = np.zeros((Bn, L, Dd))
    for t in range(L):
        a = np.exp(dt[:, t, :, None] * A[None, :, :])                  # [B, D, N]
        h = a * h + (dt[:, t, :] * u[:, t, :])[:, :, None] * B[:, t, None, :]
        o = np.einsum("bdn,bn->bd", h, C[:, t, :])
        if D is not None:
            o = o + D[None, :] * u[:, t, :]
        if z is not None:
            o = o * z[:, t, :] * _np_sigmoid(z[:, t, :])
        y[:, t, :] = o
    return y, h


def np_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None, delta_softplus=True,
           h0=None):
    """numpy backward (float64), the adjoint of ``np_fwd``."""
    u, A, B, C, D, z, x, dt = _np_prep(u, delta, A, B, C, D, z, delta_bias, delta_softplus)
    dy = _arr(dy, np.float64)
    Bn, L, Dd = u.shape
    N = A.shape[1]
    hs = np.zeros((L + 1, Bn, Dd, N))
    if h0 is not None:
        hs[0] = _arr(h0, np.float64)
    As = np.zeros((L, Bn, Dd, N))
    os_ = np.zeros((L, Bn, Dd))
    for t in range(L):
        a = np.exp(dt[:, t, :, None] * A[None, :, :])
        As[t] = a
        hs[t + 1] = a * hs[t] + (dt[:, t, :] * u[:, t, :])[:, :, None] * B[:, t, None, :]
        o = np.einsum("bdn,bn->bd", hs[t + 1], C[:, t, :])
        if D is not None:
            o = o + D[None, :] * u[:, t, :]
        os_[t] = o
    du = np.zeros((Bn, L, Dd)); ddt = np.zeros((Bn, L, Dd))
    dA = np.zeros((Dd, N)); dB = np.zeros((Bn, L, N)); dC = np.zeros((Bn, L, N))
    dD = np.zeros(Dd) if D is not None else None
    dz = np.zeros((Bn, L, Dd)) if z is not None else None
    carry = np.zeros((Bn, Dd, N))          # a_{t+1} * dL/dh_{t+1}
    for t in range(L - 1, -1, -1):
        if z is not None:
            s = _np_sigmoid(z[:, t, :])
            dz[:, t, :] = dy[:, t, :] * os_[t] * s * (1.0 + z[:, t, :] * (1.0 - s))
            g = dy[:, t, :] * z[:, t, :] * s
        else:
            g = dy[:, t, :]
        dh = carry + g[:, :, None] * C[:, t, None, :]                  # dL/dh_t
        dC[:, t, :] = np.einsum("bd,bdn->bn", g, hs[t + 1])
        dB[:, t, :] = np.einsum("bdn,bd->bn", dh, dt[:, t, :] * u[:, t, :])
        ga = dh * hs[t]                                                 # dL/da_t
        dA += np.einsum("bdn,bd->dn", ga * As[t], dt[:, t, :])
        ddt[:, t, :] = (np.einsum("bdn,dn->bd", ga * As[t], A)
                        + u[:, t, :] * np.einsum("bdn,bn->bd", dh, B[:, t, :]))
        du[:, t, :] = dt[:, t, :] * np.einsum("bdn,bn->bd", dh, B[:, t, :])
        if D is not None:
            du[:, t, :] += g * D[None, :]
            dD += np.einsum("bd,bd->d", g, u[:, t, :])
        carry = dh * As[t]
    dx = ddt * _np_sigmoid(x) if delta_softplus else ddt
    return {"du": du, "ddelta": dx, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dz": dz,
            "ddelta_bias": dx.sum(axis=(0, 1)) if delta_bias is not None else None,
            "dh0": carry if h0 is not None else None}


# Complex-valued variant (numpy, complex128): see ``oracle/cplx.py``.
from .cplx import bwd_complex, fwd_complex  # noqa: E402
