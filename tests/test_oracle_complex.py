"""Pins for the complex-valued oracle (``oracle/cplx.py``; no GPU).

The scan page (baracuda-kernels "src/attention/selective_scan.rs", module
docs, "Trailblazer scope") reserves complex variants without defining them;
the oracle takes its "Algorithm summary" recurrence with A, B, C and the state
complex and y the real part of the readout.  It is pinned against things other
than itself:

* a hand-worked step with every gradient (``golden/complex_examples.json``);
* zero imaginary parts reduce it to the real oracle (the C loop, pinned in
  ``test_oracle_pins.py``), gradients' imaginary parts being zero;
* the closed form of a constant-input scan, a geometric series in
  q = exp(dt * A);
* an O(L^2) unrolled evaluation written with real 2x2 rotation-scaling
  matrices instead of complex numbers;
* the split-sequence identity with a complex initial state;
* central finite differences of the backward in every real and imaginary
  input component.

Each check takes the implementation as an argument, so that the mutant test
at the end can run the same checks on deliberately broken copies of the
oracle source: each planted mistake must fail at least one of them.
"""
import json
import math
import os
import types

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")


def _rand_complex(seed, Bn=2, L=7, D=3, N=4, extras=True):
    """Small random complex problem (float64 (re, im) pairs)."""
    rng = np.random.default_rng(seed)
    p = {
        "u": rng.normal(size=(Bn, L, D)),
        "delta": rng.normal(-1.0, 0.5, size=(Bn, L, D)),
        "A": np.stack([-np.exp(rng.normal(size=(D, N))), rng.normal(0, 2.0, size=(D, N))], -1),
        "B": rng.normal(size=(Bn, L, N, 2)),
        "C": rng.normal(size=(Bn, L, N, 2)),
        "D": rng.normal(1.0, 0.1, size=D) if extras else None,
        "z": rng.normal(size=(Bn, L, D)) if extras else None,
        "delta_bias": rng.normal(0, 0.1, size=D) if extras else None,
    }
    h0 = rng.normal(size=(Bn, D, N, 2))
    dy = rng.normal(size=(Bn, L, D))
    return p, h0, dy


# --------------------------------------------------------------- the checks

def check_golden(fwd, bwd):
    with open(os.path.join(GOLDEN, "complex_examples.json")) as f:
        doc = json.load(f)
    for ex in doc["examples"]:
        a = {k: (None if ex[k] is None else np.array(ex[k], dtype=np.float64)) for k in KEYS}
        h0 = np.array(ex["h0"])
        y, ls = fwd(**a, delta_softplus=ex["delta_softplus"], h0=h0)
        np.testing.assert_allclose(y, ex["y"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(ls, ex["last_state"], rtol=0, atol=1e-13)
        g = bwd(**a, dy=np.array(ex["dy"]), delta_softplus=ex["delta_softplus"], h0=h0)
        for k, v in ex["grads"].items():
            np.testing.assert_allclose(g[k], v, rtol=0, atol=1e-13, err_msg=k)


def check_reduces_to_real(fwd, bwd):
    p, h0, dy = _rand_complex(11, Bn=2, L=9, D=3, N=4)
    for k in ("A", "B", "C"):
        p[k][..., 1] = 0.0
    h0[..., 1] = 0.0
    real = {k: (None if p[k] is None else (p[k][..., 0] if k in ("A", "B", "C") else p[k]))
            for k in KEYS}
    y, ls = fwd(**p, h0=h0)
    yr, lsr = oracle.fwd(**real, return_last_state=True, h0=h0[..., 0])
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls[..., 0], lsr, rtol=1e-12, atol=1e-13)
    assert np.all(ls[..., 1] == 0)
    g = bwd(**p, dy=dy, h0=h0)
    r = oracle.bwd(**real, dy=dy, h0=h0[..., 0])
    for k in ("du", "ddelta", "dD", "dz", "ddelta_bias"):
        np.testing.assert_allclose(g[k], r[k], rtol=1e-11, atol=1e-12, err_msg=k)
    for k in ("dA", "dB", "dC", "dh0"):
        np.testing.assert_allclose(g[k][..., 0], r[k], rtol=1e-11, atol=1e-12, err_msg=k)
        np.testing.assert_allclose(g[k][..., 1], 0.0, rtol=0, atol=1e-12, err_msg=k)


def check_geometric_series(fwd, bwd):
    """Constant dt, u = 1, B = 1, C fixed, one state: h_t = dt (1 - q^{t+1}) / (1 - q),
    q = exp(dt * A), y_t = Re(C h_t)."""
    L, dt = 25, 0.3
    for A in (0.7j, -0.2 + 0.7j, -1.5 - 2.0j):
        Cc = 0.5 - 0.25j
        p = {"u": np.ones((1, L, 1)), "delta": np.full((1, L, 1), dt),
             "A": np.array([[[A.real, A.imag]]]), "B": np.tile([1.0, 0.0], (1, L, 1, 1)),
             "C": np.tile([Cc.real, Cc.imag], (1, L, 1, 1)), "D": None, "z": None,
             "delta_bias": None}
        y, ls = fwd(**p, delta_softplus=False)
        q = np.exp(dt * A)
        t = np.arange(L)
        h = dt * (1 - q ** (t + 1)) / (1 - q)
        np.testing.assert_allclose(y[0, :, 0], (Cc * h).real, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ls[0, 0, 0], [h[-1].real, h[-1].imag], rtol=1e-12)


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _softplus(x):
    return np.log1p(np.exp(x))


def check_block_bruteforce(fwd, bwd):
    """y from the unrolled sum with real 2x2 matrices:
    h_t = (prod_{r<=t} M_r) h0 + sum_{s<=t} (prod_{s<r<=t} M_r) v_s, where
    M = e^{dt Re A} [[cos, -sin], [sin, cos]](dt Im A) and v_s = dt u (Re B, Im B);
    the readout is Re(C) h_re - Im(C) h_im."""
    p, h0, _ = _rand_complex(21, Bn=1, L=6, D=2, N=2)
    y, ls = fwd(**p, h0=h0)
    Bn, L, D = p["u"].shape
    N = p["A"].shape[1]
    dt = _softplus(p["delta"] + p["delta_bias"][None, None, :])
    for d in range(D):
        for t in range(L):
            o = 0.0
            for n in range(N):
                ar, ai = p["A"][d, n]

                def M(r):
                    th = dt[0, r, d] * ai
                    return math.exp(dt[0, r, d] * ar) * np.array(
                        [[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])

                h = np.eye(2)
                for r in range(t + 1):
                    h = M(r) @ h
                h = h @ h0[0, d, n]
                for s in range(t + 1):
                    P = np.eye(2)
                    for r in range(s + 1, t + 1):
                        P = M(r) @ P
                    h = h + P @ (dt[0, s, d] * p["u"][0, s, d] * p["B"][0, s, n])
                cr, ci = p["C"][0, t, n]
                o += cr * h[0] - ci * h[1]
                if t == L - 1:
                    np.testing.assert_allclose(ls[0, d, n], h, rtol=1e-12, atol=1e-13)
            o += p["D"][d] * p["u"][0, t, d]
            o *= _silu(p["z"][0, t, d])
            assert abs(y[0, t, d] - o) <= 1e-12 * max(1.0, abs(o)), (t, d, y[0, t, d], o)


def check_split_sequence(fwd, bwd):
    p, h0, _ = _rand_complex(31, Bn=2, L=12, D=3, N=3)
    y, ls = fwd(**p, h0=h0)
    s = 5
    cut = lambda lo, hi: {k: (None if p[k] is None else (p[k][:, lo:hi] if k in
                          ("u", "delta", "B", "C", "z") else p[k])) for k in KEYS}
    y1, l1 = fwd(**cut(0, s), h0=h0)
    y2, l2 = fwd(**cut(s, 12), h0=l1)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, ls, rtol=1e-13, atol=1e-14)


def check_finite_differences(fwd, bwd):
    p, h0, dy = _rand_complex(41, Bn=1, L=4, D=2, N=2)
    g = bwd(**p, dy=dy, h0=h0)
    loss = lambda q, hh: float(np.sum(dy * fwd(**q, h0=hh)[0]))
    eps = 1e-6
    names = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "z": "dz", "delta_bias": "ddelta_bias"}
    for k, gk in list(names.items()) + [("h0", "dh0")]:
        base = h0 if k == "h0" else p[k]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1, -1):
                x = base.copy()
                x[idx] += sgn * eps
                if k == "h0":
                    vals.append(loss(p, x))
                else:
                    vals.append(loss({**p, k: x}, h0))
            num[idx] = (vals[0] - vals[1]) / (2 * eps)
        np.testing.assert_allclose(g[gk], num, rtol=2e-6, atol=2e-8, err_msg=k)


CHECKS = [check_golden, check_reduces_to_real, check_geometric_series, check_block_bruteforce,
          check_split_sequence, check_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_complex_oracle(check):
    check(oracle.fwd_complex, oracle.bwd_complex)


# ---------------------------------------------------------------- mutants

_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                    "cplx.py")

# (description, text in oracle/cplx.py, replacement, occurrence to change)
MUTANTS = [
    ("readout takes the imaginary part",
     'o = np.einsum("bdn,bn->bd", h, C[:, t, :]).real', 'o = np.einsum("bdn,bn->bd", h, C[:, t, :]).imag', 1),
    ("decay uses conj(A)",
     "a = np.exp(dt[:, t, :, None] * A[None, :, :])", "a = np.exp(dt[:, t, :, None] * np.conj(A)[None, :, :])", 1),
    ("input drive uses conj(B)",
     "h = a * h + (dt[:, t, :] * u[:, t, :])[:, :, None] * B[:, t, None, :]",
     "h = a * h + (dt[:, t, :] * u[:, t, :])[:, :, None] * np.conj(B[:, t, None, :])", 1),
    ("adjoint seed without conj(C)",
     "lam = carry + g[:, :, None] * np.conj(C[:, t, None, :])", "lam = carry + g[:, :, None] * C[:, t, None, :]", 1),
    ("dC without conj(h)",
     'dC[:, t, :] = np.einsum("bd,bdn->bn", g, np.conj(hs[t + 1]))', 'dC[:, t, :] = np.einsum("bd,bdn->bn", g, hs[t + 1])', 1),
    ("dB uses conj(lam)",
     'dB[:, t, :] = np.einsum("bdn,bd->bn", lam, s_u)', 'dB[:, t, :] = np.einsum("bdn,bd->bn", np.conj(lam), s_u)', 1),
    ("dw without conj(a)",
     "dw = np.conj(As[t]) * lam * np.conj(hs[t])", "dw = As[t] * lam * np.conj(hs[t])", 1),
    ("dw uses h_t instead of h_{t-1}",
     "dw = np.conj(As[t]) * lam * np.conj(hs[t])", "dw = np.conj(As[t]) * lam * np.conj(hs[t + 1])", 1),
    ("adjoint carried with a instead of conj(a)",
     "carry = np.conj(As[t]) * lam", "carry = As[t] * lam", 1),
    ("ddt from A instead of conj(A)",
     'ddt[:, t, :] = np.einsum("bdn,dn->bd", dw, np.conj(A)).real', 'ddt[:, t, :] = np.einsum("bdn,dn->bd", dw, A).real', 1),
    ("du from B instead of conj(B)",
     'rb = np.einsum("bdn,bn->bd", lam, np.conj(B[:, t, :])).real', 'rb = np.einsum("bdn,bn->bd", lam, B[:, t, :]).real', 1),
]


def _load_mutant(old, new, occurrence):
    src = open(_SRC).read()
    pos = -1
    for _ in range(occurrence):
        pos = src.index(old, pos + 1)
    src = src[:pos] + new + src[pos + len(old):]
    mod = types.ModuleType("oracle._cplx_mutant")
    mod.__package__ = "oracle"
    exec(compile(src, "cplx_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_complex_mutant_is_caught(desc, old, new, occ):
    m = _load_mutant(old, new, occ)
    failed = []
    for check in CHECKS:
        try:
            check(m.fwd_complex, m.bwd_complex)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin catches: {desc}"
