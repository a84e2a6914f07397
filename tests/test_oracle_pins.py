"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-worked
examples, closed forms of the recurrence (A = 0, constant inputs, L = 1),
an O(L^2) unrolled formula evaluated by brute force, softplus / gate identities,
linearity, and, for the backward, central finite differences and a
dot-product (adjoint) test.  The recurrence is the "Algorithm summary" of the
baracuda-kernels page src/attention/selective_scan.rs.  The initial state h0
(the carried per-layer state of the mamba-rs page mamba_ssm/gpu/backward.rs)
is pinned by a hand-worked decode step, the split-sequence identity, a closed
form with no input drive, and finite differences.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from ss_inputs import random_inputs, WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")


def _np(inp):
    return {k: (None if inp[k] is None else inp[k].double().numpy()) for k in KEYS}


def _rand(seed, Bn=2, L=7, D=5, N=3, **kw):
    return _np(random_inputs(Bn, L, D, N, seed=seed, **kw))


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _softplus(x):
    return np.log1p(np.exp(x)) if x < 30 else x + np.log1p(np.exp(-x))


# ----------------------------------------------------------------- golden

def test_golden_hand_examples():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        doc = json.load(f)
    for ex in doc["examples"]:
        args = {k: (None if ex[k] is None else np.array(ex[k], dtype=np.float64)) for k in KEYS}
        for impl in ("c", "np"):
            if impl == "c":
                y, ls = oracle.fwd(**args, delta_softplus=ex["delta_softplus"],
                                   return_last_state=True)
            else:
                y, ls = oracle.np_fwd(**args, delta_softplus=ex["delta_softplus"])
            np.testing.assert_allclose(y, np.array(ex["y"]), rtol=1e-13, atol=1e-13,
                                       err_msg=f"{ex['name']} ({impl})")
            np.testing.assert_allclose(ls, np.array(ex["last_state"]), rtol=1e-13,
                                       atol=1e-13, err_msg=f"{ex['name']} ({impl})")


# ------------------------------------------------------- forward closed forms

def _brute_force(args, delta_softplus=True):
    """y and last state from the unrolled form
    h_t[n] = sum_{s<=t} exp(A[n] * sum_{r=s+1..t} dt_r) * dt_s * B_s[n] * u_s,
    evaluated with explicit loops."""
    u, delta, A, Bm, Cm, Dk, z, bias = (args[k] for k in KEYS)
    Bn, L, D = u.shape
    N = A.shape[1]
    y = np.zeros((Bn, L, D))
    ls = np.zeros((Bn, D, N))
    for b in range(Bn):
        for d in range(D):
            x = [delta[b, t, d] + (bias[d] if bias is not None else 0.0) for t in range(L)]
            dt = [_softplus(v) if delta_softplus else v for v in x]
            for t in range(L):
                o = 0.0
                for n in range(N):
                    h = 0.0
                    for s in range(t + 1):
                        decay = math.exp(A[d, n] * sum(dt[s + 1:t + 1]))
                        h += decay * dt[s] * Bm[b, s, n] * u[b, s, d]
                    o += Cm[b, t, n] * h
                    if t == L - 1:
                        ls[b, d, n] = h
                if Dk is not None:
                    o += Dk[d] * u[b, t, d]
                if z is not None:
                    o *= _silu(z[b, t, d])
                y[b, t, d] = o
    return y, ls


@pytest.mark.parametrize("opts", [
    dict(has_D=True, has_z=True, has_bias=True, softplus=True),
    dict(has_D=False, has_z=False, has_bias=False, softplus=True),
    dict(has_D=True, has_z=False, has_bias=True, softplus=False),
])
def test_brute_force_unrolled(opts):
    sp = opts.pop("softplus")
    args = _rand(11, Bn=2, L=6, D=3, N=4, **opts)
    if not sp:
        args["delta"] = np.abs(args["delta"])  # keep delta_eff positive without softplus
    y_ref, ls_ref = _brute_force(args, sp)
    y, ls = oracle.fwd(**args, delta_softplus=sp, return_last_state=True)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ls, ls_ref, rtol=1e-12, atol=1e-12)
    yn, lsn = oracle.np_fwd(**args, delta_softplus=sp)
    np.testing.assert_allclose(yn, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lsn, ls_ref, rtol=1e-12, atol=1e-12)


def test_A_zero_is_running_sum():
    """A = 0 gives a = 1, so h_t = sum_{s<=t} dt_s B_s u_s."""
    args = _rand(3, Bn=2, L=9, D=4, N=3, has_D=False, has_z=False, has_bias=True)
    args["A"] = np.zeros_like(args["A"])
    y, ls = oracle.fwd(**args, return_last_state=True)
    x = args["delta"] + args["delta_bias"][None, None, :]
    dt = np.log1p(np.exp(x))
    inc = (dt * args["u"])[..., None] * args["B"][:, :, None, :]      # [B, L, D, N]
    h = np.cumsum(inc, axis=1)
    y_ref = np.einsum("bldn,bln->bld", h, args["C"])
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ls, h[:, -1], rtol=1e-12, atol=1e-12)


def test_constant_inputs_geometric_series():
    """Constant dt, u, B, C over time: h_t[n] = dt B[n] u (1 - a^(t+1)) / (1 - a)."""
    Bn, L, D, N = 1, 40, 3, 4
    rng = np.random.default_rng(5)
    u0 = rng.normal(size=D)
    dl = rng.normal(-1, 0.5, size=D)
    B0 = rng.normal(size=N)
    C0 = rng.normal(size=N)
    A = -np.exp(rng.normal(size=(D, N)))
    args = dict(u=np.broadcast_to(u0, (Bn, L, D)).copy(),
                delta=np.broadcast_to(dl, (Bn, L, D)).copy(), A=A,
                B=np.broadcast_to(B0, (Bn, L, N)).copy(),
                C=np.broadcast_to(C0, (Bn, L, N)).copy(), D=None, z=None, delta_bias=None)
    y, ls = oracle.fwd(**args, return_last_state=True)
    dt = np.log1p(np.exp(dl))
    a = np.exp(dt[:, None] * A)                                         # [D, N]
    t = np.arange(L)[:, None, None]
    h = (dt * u0)[None, :, None] * B0[None, None, :] * (1 - a[None] ** (t + 1)) / (1 - a[None])
    y_ref = np.einsum("tdn,n->td", h, C0)[None]
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(ls[0], h[-1], rtol=1e-11, atol=1e-12)


def test_single_step_by_hand():
    """L = 1: y0 = (dt u sum_n B C + D u) silu(z); last_state = dt B u."""
    args = _rand(17, Bn=3, L=1, D=4, N=5)
    y, ls = oracle.fwd(**args, return_last_state=True)
    x = args["delta"][:, 0] + args["delta_bias"][None]
    dt = np.log1p(np.exp(x))                                            # [B, D]
    BC = np.sum(args["B"][:, 0] * args["C"][:, 0], axis=1)              # [B]
    u = args["u"][:, 0]
    o = dt * u * BC[:, None] + args["D"][None] * u
    np.testing.assert_allclose(y[:, 0], o * _silu(args["z"][:, 0]), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(ls, (dt * u)[:, :, None] * args["B"][:, 0][:, None, :],
                               rtol=1e-13, atol=1e-14)


def test_softplus_identities_through_the_op():
    """N = 1, A = 0, B = C = u = 1, L = 1, no D / z: y = delta_eff exactly."""
    xs = np.array([-30.0, -5.0, -0.5, 0.0, 0.5, 5.0, 30.0])
    D = xs.size

    def run(x, sp):
        return oracle.fwd(u=np.ones((1, 1, D)), delta=x.reshape(1, 1, D), A=np.zeros((D, 1)),
                          B=np.ones((1, 1, 1)), C=np.ones((1, 1, 1)), delta_softplus=sp)[0][0, 0]

    sp_pos = run(xs, True)
    sp_neg = run(-xs, True)
    assert sp_pos[3] == pytest.approx(math.log(2.0), rel=1e-15)
    np.testing.assert_allclose(sp_pos - sp_neg, xs, rtol=1e-14, atol=1e-14)
    assert np.all(sp_pos > 0)
    np.testing.assert_array_equal(run(xs, False), xs)
    # the bias adds to delta before softplus
    y = oracle.fwd(u=np.ones((1, 1, D)), delta=np.zeros((1, 1, D)), A=np.zeros((D, 1)),
                   B=np.ones((1, 1, 1)), C=np.ones((1, 1, 1)), delta_bias=xs)[0][0, 0]
    np.testing.assert_allclose(y, sp_pos, rtol=1e-15)


def test_softplus_of_inverse_softplus_bias():
    """The m130m bias is log(expm1(s)); softplus of it is s in [1e-3, 0.1]."""
    inp = make_inputs(WORKLOADS["m130m"])
    bias = inp["delta_bias"].double().numpy()
    D = bias.size
    s = oracle.fwd(u=np.ones((1, 1, D)), delta=np.zeros((1, 1, D)), A=np.zeros((D, 1)),
                   B=np.ones((1, 1, 1)), C=np.ones((1, 1, 1)), delta_bias=bias)[0][0, 0]
    assert s.min() >= 1e-3 * (1 - 1e-6) and s.max() <= 0.1 * (1 + 1e-6)


def test_gate_zero_gives_zero():
    args = _rand(23)
    args["z"] = np.zeros_like(args["z"])
    y, _ = oracle.fwd(**args)
    assert np.all(y == 0.0)


def test_linearity():
    """Without z, y is linear in u; without z and D it is linear in B and in C."""
    a = _rand(31, has_z=False, has_D=True)
    b = _rand(32, has_z=False, has_D=True)
    al, be = 0.7, -1.3
    y1 = oracle.fwd(**a)[0]
    y2 = oracle.fwd(**{**a, "u": b["u"]})[0]
    y12 = oracle.fwd(**{**a, "u": al * a["u"] + be * b["u"]})[0]
    np.testing.assert_allclose(y12, al * y1 + be * y2, rtol=1e-11, atol=1e-12)
    a["D"] = None
    for key in ("B", "C"):
        y1 = oracle.fwd(**a)[0]
        y2 = oracle.fwd(**{**a, key: b[key]})[0]
        y12 = oracle.fwd(**{**a, key: al * a[key] + be * b[key]})[0]
        np.testing.assert_allclose(y12, al * y1 + be * y2, rtol=1e-11, atol=1e-12)


def test_last_state_readout_consistency():
    """Without z: y[L-1] = sum_n C[L-1, n] last_state[n] + D u[L-1]."""
    a = _rand(41, Bn=2, L=13, D=6, N=5, has_z=False)
    y, ls = oracle.fwd(**a, return_last_state=True)
    ref = np.einsum("bdn,bn->bd", ls, a["C"][:, -1]) + a["D"][None] * a["u"][:, -1]
    np.testing.assert_allclose(y[:, -1], ref, rtol=1e-12, atol=1e-13)


def test_channel_subset_matches_full():
    a = _rand(43, Bn=3, L=17, D=9, N=4)
    y, ls = oracle.fwd(**a, return_last_state=True)
    cb, cd = [0, 2, 1, 2], [0, 8, 4, 3]
    ys, lss = oracle.fwd_channels(**a, chan_b=cb, chan_d=cd)
    for i, (b, d) in enumerate(zip(cb, cd)):
        np.testing.assert_array_equal(ys[i], y[b, :, d])
        np.testing.assert_array_equal(lss[i], ls[b, d])


def test_threads_do_not_change_forward():
    a = _rand(47, Bn=2, L=20, D=13, N=4)
    y1 = oracle.fwd(**a, nthreads=1)[0]
    y5 = oracle.fwd(**a, nthreads=5)[0]
    np.testing.assert_array_equal(y1, y5)


def test_c_matches_numpy_forward():
    for seed, opts in [(51, {}), (52, dict(has_D=False, has_z=False, has_bias=False))]:
        a = _rand(seed, Bn=2, L=33, D=7, N=6, **opts)
        y, ls = oracle.fwd(**a, return_last_state=True)
        yn, lsn = oracle.np_fwd(**a)
        np.testing.assert_allclose(y, yn, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ls, lsn, rtol=1e-12, atol=1e-13)


def test_degenerate_shapes():
    # N = 0: no state, y = D u silu(z)
    a = _rand(61, Bn=2, L=5, D=3, N=1)
    a["A"] = a["A"][:, :0]
    a["B"] = a["B"][:, :, :0]
    a["C"] = a["C"][:, :, :0]
    y, ls = oracle.fwd(**a, return_last_state=True)
    np.testing.assert_allclose(y, a["D"][None, None] * a["u"] * _silu(a["z"]), rtol=1e-15)
    assert ls.shape == (2, 3, 0)
    # L = 0: nothing to compute; the final state is the initial zero state
    a = _rand(62, Bn=2, L=1, D=3, N=2)
    for k in ("u", "delta", "z"):
        a[k] = a[k][:, :0]
    for k in ("B", "C"):
        a[k] = a[k][:, :0]
    y, ls = oracle.fwd(**a, return_last_state=True)
    assert y.shape == (2, 0, 3)
    np.testing.assert_array_equal(ls, np.zeros((2, 3, 2)))


# ----------------------------------------------------------------- backward

GRAD_OF = {"u": "du", "delta": "ddelta", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "z": "dz", "delta_bias": "ddelta_bias"}


def _loss(args, dy, sp):
    return float(np.sum(oracle.fwd(**args, delta_softplus=sp)[0] * dy))


@pytest.mark.parametrize("sp,opts", [
    (True, dict(has_D=True, has_z=True, has_bias=True)),
    (False, dict(has_D=False, has_z=False, has_bias=True)),
    (True, dict(has_D=True, has_z=False, has_bias=False)),
])
def test_backward_finite_differences(sp, opts):
    a = _rand(71, Bn=2, L=5, D=3, N=4, **opts)
    if not sp:  # keep delta_eff positive and moderate without softplus
        a["delta"] = np.abs(a["delta"]) * 0.5
        if a["delta_bias"] is not None:
            a["delta_bias"] = np.abs(a["delta_bias"]) * 0.01
    dy = np.random.default_rng(72).normal(size=a["u"].shape)
    g = oracle.bwd(**a, dy=dy, delta_softplus=sp)
    for k in KEYS:
        if a[k] is None:
            assert g[GRAD_OF[k]] is None
            continue
        fd = np.zeros_like(a[k])
        it = np.nditer(a[k], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = a[k][idx]
            eps = 1e-6 * max(1.0, abs(x0))
            ap = {**a, k: a[k].copy()}
            ap[k][idx] = x0 + eps
            am = {**a, k: a[k].copy()}
            am[k][idx] = x0 - eps
            fd[idx] = (_loss(ap, dy, sp) - _loss(am, dy, sp)) / (2 * eps)
        np.testing.assert_allclose(g[GRAD_OF[k]], fd, rtol=2e-6, atol=2e-7,
                                   err_msg=f"gradient of {k}")


def test_backward_dot_product():
    """<dy, J v> (directional derivative by central differences) = <J^T dy, v>."""
    a = _rand(81, Bn=2, L=11, D=4, N=5)
    rng = np.random.default_rng(82)
    dy = rng.normal(size=a["u"].shape)
    v = {k: rng.normal(size=a[k].shape) for k in KEYS}
    g = oracle.bwd(**a, dy=dy)
    eps = 1e-6
    lp = _loss({k: a[k] + eps * v[k] for k in KEYS}, dy, True)
    lm = _loss({k: a[k] - eps * v[k] for k in KEYS}, dy, True)
    lhs = (lp - lm) / (2 * eps)
    rhs = sum(float(np.sum(g[GRAD_OF[k]] * v[k])) for k in KEYS)
    assert lhs == pytest.approx(rhs, rel=1e-7)


def test_backward_identities():
    a = _rand(91, Bn=3, L=9, D=5, N=4)
    dy = np.random.default_rng(92).normal(size=a["u"].shape)
    g = oracle.bwd(**a, dy=dy)
    # ddelta_bias is the (b, t) sum of ddelta
    np.testing.assert_allclose(g["ddelta_bias"], g["ddelta"].sum(axis=(0, 1)), rtol=1e-12)
    # dD = sum_{b,t} g u with g = dy * silu(z)
    gg = dy * _silu(a["z"])
    np.testing.assert_allclose(g["dD"], np.sum(gg * a["u"], axis=(0, 1)), rtol=1e-12)
    # without z the gradient reaching the readout is dy itself
    a2 = {**a, "z": None}
    g2 = oracle.bwd(**a2, dy=dy)
    np.testing.assert_allclose(g2["dD"], np.sum(dy * a["u"], axis=(0, 1)), rtol=1e-12)
    # with L = 1 the decay never acts (h_{-1} = 0), so dA = 0 exactly
    a1 = {k: (None if a[k] is None else (a[k][:, :1] if a[k].ndim == 3 else a[k])) for k in KEYS}
    g1 = oracle.bwd(**a1, dy=dy[:, :1])
    assert np.all(g1["dA"] == 0.0)


def test_backward_c_matches_numpy():
    for seed, opts in [(95, {}), (96, dict(has_D=False, has_z=False, has_bias=False))]:
        a = _rand(seed, Bn=2, L=21, D=6, N=5, **opts)
        dy = np.random.default_rng(seed + 1).normal(size=a["u"].shape)
        gc = oracle.bwd(**a, dy=dy, nthreads=3)
        gn = oracle.np_bwd(**a, dy=dy)
        for k, v in gc.items():
            if v is None:
                assert gn[k] is None
            else:
                np.testing.assert_allclose(v, gn[k], rtol=1e-11, atol=1e-12, err_msg=k)


# ------------------------------------------------------------ initial state

def _h0(args, seed):
    Bn, L, D = args["u"].shape
    N = args["A"].shape[1]
    return np.random.default_rng(seed).normal(size=(Bn, D, N))


def test_h0_golden_decode_step():
    with open(os.path.join(GOLDEN, "h0_examples.json")) as f:
        doc = json.load(f)
    for ex in doc["examples"]:
        args = {k: (None if ex[k] is None else np.array(ex[k], dtype=np.float64)) for k in KEYS}
        h0 = np.array(ex["h0"])
        dy = np.array(ex["dy"])
        for impl in ("c", "np"):
            if impl == "c":
                y, ls = oracle.fwd(**args, delta_softplus=ex["delta_softplus"],
                                   return_last_state=True, h0=h0)
                g = oracle.bwd(**args, dy=dy, delta_softplus=ex["delta_softplus"], h0=h0)
            else:
                y, ls = oracle.np_fwd(**args, delta_softplus=ex["delta_softplus"], h0=h0)
                g = oracle.np_bwd(**args, dy=dy, delta_softplus=ex["delta_softplus"], h0=h0)
            np.testing.assert_allclose(y, np.array(ex["y"]), rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(ls, np.array(ex["last_state"]), rtol=1e-13, atol=1e-13)
            for k, v in ex["grads"].items():
                np.testing.assert_allclose(g[k], np.array(v), rtol=1e-13, atol=1e-13,
                                           err_msg=f"{ex['name']} {k} ({impl})")


@pytest.mark.parametrize("split", [1, 6, 13])
def test_h0_split_sequence(split):
    """Running t < s, then t >= s from the state reached at s, is the same
    recurrence as one run (outputs and final state)."""
    a = _rand(301, Bn=2, L=19, D=4, N=5)
    h0 = _h0(a, 302)
    y, ls = oracle.fwd(**a, return_last_state=True, h0=h0)
    first = {k: (v[:, :split] if v is not None and v.ndim == 3 else v) for k, v in a.items()}
    second = {k: (v[:, split:] if v is not None and v.ndim == 3 else v) for k, v in a.items()}
    y1, ls1 = oracle.fwd(**first, return_last_state=True, h0=h0)
    y2, ls2 = oracle.fwd(**second, return_last_state=True, h0=ls1)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ls2, ls, rtol=1e-12, atol=1e-13)


def test_h0_closed_form_without_input():
    """With B = 0 the state only decays: h_t = exp(A * sum_{s<=t} dt_s) h0."""
    a = _rand(311, Bn=2, L=9, D=3, N=4, has_D=False, has_z=False)
    a["B"] = np.zeros_like(a["B"])
    h0 = _h0(a, 312)
    y, ls = oracle.fwd(**a, return_last_state=True, h0=h0)
    x = a["delta"] + a["delta_bias"][None, None, :]
    dt = np.vectorize(_softplus)(x)
    cum = np.cumsum(dt, axis=1)                                     # [B, L, D]
    hs = np.exp(cum[..., None] * a["A"][None, None]) * h0[:, None]  # [B, L, D, N]
    yr = np.einsum("bldn,bln->bld", hs, a["C"])
    np.testing.assert_allclose(y, yr, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ls, hs[:, -1], rtol=1e-12, atol=1e-14)


def test_h0_finite_differences_and_numpy():
    a = _rand(321, Bn=2, L=5, D=3, N=4)
    h0 = _h0(a, 322)
    dy = np.random.default_rng(323).normal(size=a["u"].shape)
    g = oracle.bwd(**a, dy=dy, h0=h0)
    fd = np.zeros_like(h0)
    it = np.nditer(h0, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        eps = 1e-6 * max(1.0, abs(h0[idx]))
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += eps
        hm[idx] -= eps
        lp = float(np.sum(oracle.fwd(**a, h0=hp)[0] * dy))
        lm = float(np.sum(oracle.fwd(**a, h0=hm)[0] * dy))
        fd[idx] = (lp - lm) / (2 * eps)
    np.testing.assert_allclose(g["dh0"], fd, rtol=2e-6, atol=2e-7)
    # the other gradients see h0 through the recurrence: finite differences in A
    fda = np.zeros_like(a["A"])
    it = np.nditer(a["A"], flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        eps = 1e-6 * max(1.0, abs(a["A"][idx]))
        ap, am = {**a, "A": a["A"].copy()}, {**a, "A": a["A"].copy()}
        ap["A"][idx] += eps
        am["A"][idx] -= eps
        lp = float(np.sum(oracle.fwd(**ap, h0=h0)[0] * dy))
        lm = float(np.sum(oracle.fwd(**am, h0=h0)[0] * dy))
        fda[idx] = (lp - lm) / (2 * eps)
    np.testing.assert_allclose(g["dA"], fda, rtol=2e-6, atol=2e-7)
    gn = oracle.np_bwd(**a, dy=dy, h0=h0)
    for k, v in g.items():
        if v is None:
            assert gn[k] is None
        else:
            np.testing.assert_allclose(v, gn[k], rtol=1e-11, atol=1e-12, err_msg=k)
    yn, lsn = oracle.np_fwd(**a, h0=h0)
    yc, lsc = oracle.fwd(**a, h0=h0, return_last_state=True)
    np.testing.assert_allclose(yc, yn, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lsc, lsn, rtol=1e-12, atol=1e-13)


def test_h0_zero_is_no_h0():
    a = _rand(331)
    z0 = np.zeros((2, 5, 3))
    y0, l0 = oracle.fwd(**a, return_last_state=True)
    y1, l1 = oracle.fwd(**a, return_last_state=True, h0=z0)
    assert np.array_equal(y0, y1) and np.array_equal(l0, l1)
    dy = np.random.default_rng(332).normal(size=a["u"].shape)
    g0 = oracle.bwd(**a, dy=dy)
    g1 = oracle.bwd(**a, dy=dy, h0=z0)
    for k in g0:
        if g0[k] is not None:
            assert np.array_equal(g0[k], g1[k]), k


# ------------------------------------------------------- packed sequences

def test_varlen_equal_lengths_match_the_dense_batch():
    a = _rand(341, Bn=3, L=11, D=4, N=5)
    h0 = _h0(a, 342)
    dy = np.random.default_rng(343).normal(size=a["u"].shape)
    pack = lambda x: None if x is None else (x.reshape(-1, x.shape[-1]) if x.ndim == 3 else x)
    p = {k: pack(v) for k, v in a.items()}
    cu = [0, 11, 22, 33]
    y, ls = oracle.fwd(**a, return_last_state=True, h0=h0)
    yv, lsv = oracle.fwd_varlen(**p, cu_seqlens=cu, h0=h0)
    np.testing.assert_allclose(yv, y.reshape(33, 4), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lsv, ls, rtol=1e-14, atol=1e-15)
    g = oracle.bwd(**a, dy=dy, h0=h0)
    gv = oracle.bwd_varlen(**p, dy=dy.reshape(33, 4), cu_seqlens=cu, h0=h0)
    for k in ("du", "ddelta", "dB", "dC", "dz"):
        np.testing.assert_allclose(gv[k], g[k].reshape(33, -1), rtol=1e-13, atol=1e-14, err_msg=k)
    for k in ("dA", "dD", "ddelta_bias", "dh0"):
        np.testing.assert_allclose(gv[k], g[k], rtol=1e-12, atol=1e-13, err_msg=k)


def test_varlen_sequences_are_independent():
    """Changing one sequence's rows leaves every other sequence's outputs alone,
    and an empty sequence returns its initial state."""
    rng = np.random.default_rng(351)
    a = _rand(352, Bn=1, L=20, D=3, N=4)
    p = {k: (None if v is None else (v[0] if v.ndim == 3 else v)) for k, v in a.items()}
    cu = [0, 6, 6, 13, 20]
    h0 = rng.normal(size=(4, 3, 4))
    y, ls = oracle.fwd_varlen(**p, cu_seqlens=cu, h0=h0)
    q = {**p, "u": p["u"].copy()}
    q["u"][6:13] += 1.0
    y2, ls2 = oracle.fwd_varlen(**q, cu_seqlens=cu, h0=h0)
    assert np.array_equal(y[:6], y2[:6]) and np.array_equal(y[13:], y2[13:])
    assert not np.allclose(y[6:13], y2[6:13])
    assert np.array_equal(ls[[0, 1, 3]], ls2[[0, 1, 3]])
    np.testing.assert_array_equal(ls[1], h0[1])


def test_f32_floor_is_close():
    """The float build of the same loop stays near the double one (diagnostic)."""
    a = _rand(99, Bn=2, L=256, D=8, N=16)
    y64 = oracle.fwd(**a)[0]
    y32 = oracle.fwd_f32(**a)[0]
    err = np.max(np.abs(y32 - y64)) / np.sqrt(np.mean(y64 ** 2))
    assert err < 1e-5


def _rel(x, r):
    """max |x - r| / max(|r|, rms(r)) over a tensor."""
    rms = float(np.sqrt(np.mean(r * r)))
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms)))


# Shapes short enough that every output is well conditioned in single
# precision: each step rounds a few times at 2^-24 ~ 6e-8 relative, so over
# L <= 64 steps the float loop stays within ~1e-6 of the double one (measured
# 1e-7 .. 2.3e-6); F32_BOUND = 2e-5 leaves a margin of about 10, while any
# mistake in the loop (a dropped term, a wrong sign or index) moves some
# output by far more than 1e-3.
F32_BOUND = 2e-5


@pytest.mark.parametrize("sp", [True, False])
@pytest.mark.parametrize("seed,shape", [(1, (2, 24, 6, 4)), (2, (1, 40, 5, 8)),
                                        (3, (2, 16, 7, 16)), (4, (1, 64, 3, 2))])
def test_f32_build_tracks_f64(seed, shape, sp):
    """The float instantiation of the loop (fwd_f32 / bwd_f32, the single-
    precision floor) against the pinned double one, every output including the
    initial-state gradient, with and without softplus."""
    Bn, L, D, N = shape
    a = _rand(700 + seed, Bn=Bn, L=L, D=D, N=N)
    if not sp:  # keep dt positive without softplus (a decaying recurrence)
        a["delta"] = np.abs(a["delta"]) * 0.3
        a["delta_bias"] = np.abs(a["delta_bias"]) * 0.01
    rng = np.random.default_rng(710 + seed)
    dy = rng.normal(size=(Bn, L, D)).astype(np.float32).astype(np.float64)
    h0 = rng.normal(size=(Bn, D, N)).astype(np.float32).astype(np.float64)
    y, ls = oracle.fwd(**a, delta_softplus=sp, return_last_state=True, h0=h0)
    y3, ls3 = oracle.fwd_f32(**a, delta_softplus=sp, return_last_state=True, h0=h0)
    assert y3.dtype == np.float32
    errs = {"y": _rel(y3, y), "last_state": _rel(ls3, ls)}
    g = oracle.bwd(**a, dy=dy, delta_softplus=sp, h0=h0)
    g3 = oracle.bwd_f32(**a, dy=dy, delta_softplus=sp, h0=h0)
    for k, v in g.items():
        assert (v is None) == (g3[k] is None), k
        if v is not None:
            assert g3[k].dtype == np.float32, k
            errs[k] = _rel(g3[k], v)
    bad = {k: e for k, e in errs.items() if not e <= F32_BOUND}
    assert not bad, bad
