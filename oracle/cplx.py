"""CPU oracle for the complex-valued selective scan (float64 / complex128).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the bench's CPU-baseline leg may use it, and it
shares no code with the HIP library.

The scan page (baracuda-kernels "src/attention/selective_scan.rs", module
docs, "Trailblazer scope") names complex variants only as reserved and
deferred.  The operation here is the same recurrence as its "Algorithm
summary" with A, B, C and the state complex and everything else real:

    x  = delta[b,t,d] + delta_bias[d],   dt = softplus(x) or x      (real)
    a  = exp(dt * A[d,n])                                           (complex)
    h  = a * h + dt * u[b,t,d] * B[b,t,n]      (h = h0 or 0 before t = 0)
    o  = Re(sum_n C[b,t,n] * h[n]) + D[d] * u[b,t,d]                (real)
    y  = o * z * sigmoid(z)                                         (z optional)

Reading: the output is the real part of the complex readout.  (A convention
that keeps one state of each conjugate pair and doubles the real part is the
same operation with C scaled by 2, which is exact in floating point.)

Storage: every complex tensor is float pairs (re, im) in its last axis: A
[D, N, 2], B / C [B, L, N, 2], h0 / last_state [B, D, N, 2].  Gradients of a
complex input are returned in the same layout as (dL/dRe, dL/dIm).

The backward is the chain-rule adjoint of the forward, worked in real terms
(a complex number as a pair of reals; ``lam`` is dL/dRe(h) + i dL/dIm(h)):

    lam_t     = g_t * conj(C_t) + conj(a_{t+1}) * lam_{t+1}
    dB_t      = dt_t u_t lam_t                 dC_t = g_t conj(h_t)
    dw_t      = conj(a_t) lam_t conj(h_{t-1})  (w = dt * A, a = exp(w))
    dA       += dt_t dw_t                      ddt_t = sum_n Re(conj(A) dw_t)
                                                        + u_t sum_n Re(conj(B_t) lam_t)
    du_t      = dt_t sum_n Re(conj(B_t) lam_t) + D g_t
    dh0       = conj(a_0) lam_0

with g the gradient reaching o (dy, through the gate when z is given); the
real-valued remainder (softplus, gate, skip) is the same as the real scan.
"""
from __future__ import annotations

import numpy as np

from . import _arr, _np_sigmoid, _np_softplus


def _c(x):
    """(…, 2) float pairs -> complex128 (None passes through)."""
    if x is None:
        return None
    a = _arr(x, np.float64)
    assert a.shape[-1] == 2, "complex tensors are (re, im) pairs in the last axis"
    return a[..., 0] + 1j * a[..., 1]


def _pairs(z):
    return np.stack([z.real, z.imag], axis=-1)


def _prep(u, delta, A, B, C, D, z, delta_bias, delta_softplus):
    u, delta, D, z, bias = [_arr(t, np.float64) for t in (u, delta, D, z, delta_bias)]
    A, B, C = _c(A), _c(B), _c(C)
    x = delta + (bias[None, None, :] if bias is not None else 0.0)
    dt = _np_softplus(x) if delta_softplus else x
    return u, A, B, C, D, z, x, dt


def fwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                h0=None):
    """Complex forward.  Returns (y [B, L, D], last_state [B, D, N, 2])."""
    u, A, B, C, D, z, x, dt = _prep(u, delta, A, B, C, D, z, delta_bias, delta_softplus)
    Bn, L, Dd = u.shape
    N = A.shape[1]
    h = np.zeros((Bn, Dd, N), dtype=np.complex128) if h0 is None else _c(h0).copy()
    y = np.zeros((Bn, L, Dd))
    for t in range(L):
        a = np.exp(dt[:, t, :, None] * A[None, :, :])                       # [B, D, N]
        h = a * h + (dt[:, t, :] * u[:, t, :])[:, :, None] * B[:, t, None, :]
        o = np.einsum("bdn,bn->bd", h, C[:, t, :]).real
        if D is not None:
            o = o + D[None, :] * u[:, t, :]
        if z is not None:
            o = o * z[:, t, :] * _np_sigmoid(z[:, t, :])
        y[:, t, :] = o
    return y, _pairs(h)


def bwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None,
                delta_softplus=True, h0=None):
    """Complex backward for the loss sum(dy * y): a dict with du, ddelta, dA,
    dB, dC, dD, dz, ddelta_bias, dh0 (complex ones as (re, im) pairs)."""
    u, A, B, C, D, z, x, dt = _prep(u, delta, A, B, C, D, z, delta_bias, delta_softplus)
    dy = _arr(dy, np.float64)
    Bn, L, Dd = u.shape
    N = A.shape[1]
    hs = np.zeros((L + 1, Bn, Dd, N), dtype=np.complex128)   # hs[t + 1] = h_t
    if h0 is not None:
        hs[0] = _c(h0)
    As = np.zeros((L, Bn, Dd, N), dtype=np.complex128)
    os_ = np.zeros((L, Bn, Dd))
    for t in range(L):
        a = np.exp(dt[:, t, :, None] * A[None, :, :])
        As[t] = a
        hs[t + 1] = a * hs[t] + (dt[:, t, :] * u[:, t, :])[:, :, None] * B[:, t, None, :]
        o = np.einsum("bdn,bn->bd", hs[t + 1], C[:, t, :]).real
        if D is not None:
            o = o + D[None, :] * u[:, t, :]
        os_[t] = o
    du = np.zeros((Bn, L, Dd)); ddt = np.zeros((Bn, L, Dd))
    dA = np.zeros((Dd, N), dtype=np.complex128)
    dB = np.zeros((Bn, L, N), dtype=np.complex128)
    dC = np.zeros((Bn, L, N), dtype=np.complex128)
    dD = np.zeros(Dd) if D is not None else None
    dz = np.zeros((Bn, L, Dd)) if z is not None else None
    carry = np.zeros((Bn, Dd, N), dtype=np.complex128)     # conj(a_{t+1}) * lam_{t+1}
    for t in range(L - 1, -1, -1):
        if z is not None:
            s = _np_sigmoid(z[:, t, :])
            dz[:, t, :] = dy[:, t, :] * os_[t] * s * (1.0 + z[:, t, :] * (1.0 - s))
            g = dy[:, t, :] * z[:, t, :] * s
        else:
            g = dy[:, t, :]
        lam = carry + g[:, :, None] * np.conj(C[:, t, None, :])            # dL/dh_t
        dC[:, t, :] = np.einsum("bd,bdn->bn", g, np.conj(hs[t + 1]))
        s_u = dt[:, t, :] * u[:, t, :]
        dB[:, t, :] = np.einsum("bdn,bd->bn", lam, s_u)
        dw = np.conj(As[t]) * lam * np.conj(hs[t])                          # dL/dw_t
        dA += np.einsum("bdn,bd->dn", dw, dt[:, t, :])
        rb = np.einsum("bdn,bn->bd", lam, np.conj(B[:, t, :])).real         # sum Re(conj(B) lam)
        ddt[:, t, :] = np.einsum("bdn,dn->bd", dw, np.conj(A)).real + u[:, t, :] * rb
        du[:, t, :] = dt[:, t, :] * rb
        if D is not None:
            du[:, t, :] += g * D[None, :]
            dD += np.einsum("bd,bd->d", g, u[:, t, :])
        carry = np.conj(As[t]) * lam
    dx = ddt * _np_sigmoid(x) if delta_softplus else ddt
    return {"du": du, "ddelta": dx, "dA": _pairs(dA), "dB": _pairs(dB), "dC": _pairs(dC),
            "dD": dD, "dz": dz,
            "ddelta_bias": dx.sum(axis=(0, 1)) if delta_bias is not None else None,
            "dh0": _pairs(carry) if h0 is not None else None}
