"""GPU parity: the HIP library against the CPU oracle (needs an MI355X).

Every call goes through the C ABI (mamba_selective_scan_02_amd wraps it with
ctypes).  Outputs are compared element by element with the float64 oracle on
the same seeded inputs; the bound is the one the target states (1e-5 f32,
2e-2 f16/bf16) on max |x - r| / max(|r|, rms(r)).  The five workloads run
in the schedule the bench times (chunk_len = 0) and are compared in full.
"""
import os

import numpy as np
import pytest
import torch

import mamba_selective_scan_02_amd as ss
import oracle
from ss_inputs import WORKLOADS, make_inputs, random_inputs
from tests.parity_util import GRADS, KEYS, TOL, rel_err, say, to_dev, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ss.load_library()
    yield


def _run_fwd(inp, sp=True, chunk_len=0, last_state=True):
    d = to_dev(inp)
    y, ls = ss.fwd(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["delta_bias"],
                   delta_softplus=sp, return_last_state=last_state, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return y, ls


def _check_fwd(inp, sp=True, chunk_len=0, tol=None, label=""):
    say("fwd", label, tuple(inp["u"].shape), inp["A"].shape[1], inp["u"].dtype, "chunk", chunk_len)
    y, ls = _run_fwd(inp, sp, chunk_len)
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, delta_softplus=sp, return_last_state=True)
    tol = tol or TOL[inp["u"].dtype]
    e_y, e_s = rel_err(to_np(y), yr), rel_err(to_np(ls), lsr)
    assert e_y <= tol, f"{label} y err {e_y:.3e} > {tol}"
    assert e_s <= max(tol, TOL[inp["A"].dtype]), f"{label} last_state err {e_s:.3e}"
    return e_y


# ------------------------------------------------------------------ forward

SHAPES = [  # (B, L, D, N)
    (1, 1, 1, 1), (1, 2, 31, 4), (3, 63, 64, 16), (2, 64, 65, 16), (1, 65, 300, 16),
    (2, 1000, 33, 16), (1, 300, 257, 8), (2, 129, 70, 17), (1, 77, 40, 32), (1, 50, 20, 64),
    (1, 40, 20, 65), (1, 33, 10, 128), (1, 21, 9, 200), (1, 19, 7, 256), (2, 17, 5, 3),
    # 8 states per lane (N = 33 .. 64), chunked: several stages, ragged tails, padded states
    (2, 600, 72, 64), (1, 300, 40, 48),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_shapes_f32(shape):
    Bn, L, D, N = shape
    _check_fwd(random_inputs(Bn, L, D, N, seed=hash(shape) % 10000), label=str(shape))


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100])
def test_fwd_forced_chunks(chunk):
    inp = random_inputs(2, 700, 96, 16, seed=77)
    _check_fwd(inp, chunk_len=chunk, label=f"chunk{chunk}")


@pytest.mark.parametrize("combo", range(16))
def test_fwd_optional_combinations(combo):
    has_D, has_z, has_bias, sp = [bool(combo >> i & 1) for i in range(4)]
    inp = random_inputs(2, 150, 70, 16, seed=200 + combo, has_D=has_D, has_z=has_z,
                        has_bias=has_bias)
    if not sp:  # keep delta_eff positive without softplus
        inp["delta"] = inp["delta"].abs() * 0.3
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    for chunk in (0, 32):
        _check_fwd(inp, sp=sp, chunk_len=chunk, label=f"combo{combo}/chunk{chunk}")


@pytest.mark.parametrize("io,pa", [("bf16", "f32"), ("f16", "f32"), ("bf16", "bf16"),
                                   ("f16", "f16")])
@pytest.mark.parametrize("N", [16, 5, 64])
def test_fwd_half_dtypes(io, pa, N):
    inp = random_inputs(2, 200, 130, N, seed=300 + N, io_dtype=io, param_dtype=pa)
    for chunk in (0, 48):
        _check_fwd(inp, chunk_len=chunk, label=f"{io}/{pa}/N{N}/chunk{chunk}")


def _offset_copy(x, elems=1):
    """x's values in a view that starts `elems` elements past an aligned address."""
    big = torch.empty(x.numel() + elems, dtype=x.dtype, device=x.device)
    big[elems:] = x.reshape(-1)
    return big[elems:].view_as(x)


@pytest.mark.parametrize("io", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N", [8, 16, 32, 64])
def test_fwd_wide_path(io, N):
    """Rows of a multiple of 16 bytes with N = 8, 16, 32, 64 take the LDS-staged
    kernel (D = 72: two full channel blocks and a partial one; L = 150: partial
    stages).  It must match the oracle, and match bit for bit the element-wise
    kernel that misaligned inputs take, since both do the same arithmetic."""
    inp = random_inputs(2, 150, 72, N, seed=450 + N, io_dtype=io)
    d = to_dev(inp)
    args = [d[k] for k in KEYS]
    for chunk in (0, 24, 100):
        _check_fwd(inp, chunk_len=chunk, label=f"wide {io}/N{N}/chunk{chunk}")
        y1, l1 = ss.fwd(*args, return_last_state=True, chunk_len=chunk)
        mis = list(args)
        mis[0] = _offset_copy(args[0])
        y2, l2 = ss.fwd(*mis, return_last_state=True, chunk_len=chunk)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(l1, l2), f"{io}/N{N}/chunk{chunk}"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fwd_chunk_fixup_exit(io):
    """The chunked LDS-staged forward reruns each chunk from its carried state
    only until every state of the workgroup equals, bit for bit, the state of
    the pass that ran the chunk from zero.  Channels whose states forget fast
    (A = -4 (n+1)) sit beside channels that never forget (A = 0) in different
    waves and lanes of the same workgroups (32 channels each), so an exit vote
    that missed one lane or one wave would leave the zero-start outputs in the
    tails of their chunks.  With h0, chunk 0 is rerun as well."""
    inp = random_inputs(1, 600, 64, 16, seed=470, io_dtype=io)
    A = inp["A"].clone()
    n = torch.arange(1, 17, dtype=A.dtype)
    A[:] = -4.0 * n
    for d in (5, 30, 33, 63):               # waves 0 and 3 of block 0, waves 0 and 3 of block 1
        A[d] = 0.0
    inp["A"] = A
    h0 = _state(inp, 471)
    d = to_dev(inp)
    for chunk in (100, 256):
        for with_h0 in (False, True):
            say("fwd fixup", io, "chunk", chunk, "h0", with_h0)
            y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True, chunk_len=chunk,
                           h0=h0.to(DEV) if with_h0 else None)
            torch.cuda.synchronize()
            yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True,
                                 h0=h0 if with_h0 else None)
            tol = TOL[inp["u"].dtype]
            assert rel_err(to_np(y), yr) <= tol, f"y chunk {chunk} h0 {with_h0}"
            assert rel_err(to_np(ls), lsr) <= max(tol, TOL[inp["A"].dtype])


def test_fwd_misaligned_16bit_rows():
    """bf16 B / C at an odd element offset take the element-wise load path."""
    inp = random_inputs(1, 40, 64, 16, seed=401, io_dtype="bf16")
    d = to_dev(inp)
    Bbig = torch.empty(d["B"].numel() + 1, dtype=torch.bfloat16, device=DEV)
    Bbig[1:] = d["B"].reshape(-1)
    Bv = Bbig[1:].view_as(d["B"])
    assert Bv.data_ptr() % 4 == 2
    y, _ = ss.fwd(d["u"], d["delta"], d["A"], Bv, d["C"], d["D"], d["z"], d["delta_bias"])
    yr, _ = oracle.fwd(**{k: inp[k] for k in KEYS})
    assert rel_err(to_np(y), yr) <= 2e-2


def test_fwd_degenerate():
    # N = 0: y = D u silu(z)
    inp = random_inputs(2, 30, 40, 1, seed=501)
    inp["A"], inp["B"], inp["C"] = inp["A"][:, :0], inp["B"][:, :, :0], inp["C"][:, :, :0]
    _check_fwd(inp, label="N0")
    # L = 0 with last_state: zeros
    inp = random_inputs(2, 1, 40, 16, seed=502)
    for k in ("u", "delta", "z", "B", "C"):
        inp[k] = inp[k][:, :0].contiguous()
    y, ls = _run_fwd(inp)
    assert y.shape == (2, 0, 40) and torch.all(ls == 0)
    # B = 0, D = 0: nothing to do
    for shp in ((0, 10, 8, 4), (2, 10, 0, 4)):
        inp = random_inputs(*shp, seed=503)
        y, ls = _run_fwd(inp)
        assert y.numel() == 0


def test_extreme_inputs():
    """Softplus and decay extremes: pre-softplus delta at +-30 (dt = 30, a
    state reset each step; dt ~ 1e-13, a state held), A = 0 on some states
    (a running sum), u = 0 on some channels: forward and backward against
    the oracle."""
    Bn, L, D, N = 2, 97, 40, 16
    inp = random_inputs(Bn, L, D, N, seed=5101, backward=True)
    g = torch.Generator().manual_seed(5102)
    pick = torch.randint(0, 5, (Bn, L, D), generator=g)
    vals = torch.tensor([-30.0, -10.0, 0.0, 10.0, 30.0], dtype=torch.float64)
    inp["delta"] = vals[pick].to(inp["delta"].dtype)
    inp["delta_bias"] = torch.zeros_like(inp["delta_bias"])
    A = inp["A"].clone()
    A[:, ::4] = 0.0
    inp["A"] = A
    u = inp["u"].clone()
    u[:, :, ::5] = 0.0
    inp["u"] = u
    h0 = _state(inp, 5103)
    d = to_dev(inp)
    for chunk in (0, 16):
        say("extreme inputs, chunk", chunk)
        y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True, chunk_len=chunk,
                       h0=h0.to(DEV))
        gr = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
        torch.cuda.synchronize()
        yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
        r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
        assert rel_err(to_np(y), yr) <= 1e-5
        assert rel_err(to_np(ls), lsr) <= 1e-5
        for k in GRADS + ("dh0",):
            if r[k] is not None:
                e = rel_err(to_np(gr[k]), r[k])
                assert e <= 1e-5, f"{k} chunk {chunk}: {e:.3e}"


def test_fwd_workloads_tiny_and_m130m():
    for name in ("tiny", "m130m"):
        w = WORKLOADS[name]
        inp = make_inputs(w)
        say("workload", name)
        _check_fwd(inp, label=name)


@pytest.mark.parametrize("name", ["m2p8b", "long"])
def test_fwd_workloads_full(name):
    """The Mamba-2.8B-shaped (bf16) and the long-sequence workloads, every
    element of y and of last_state against the float64 oracle, in the schedule
    the bench times (single pass for the 2.8B shape, 128 chunks for the long
    one)."""
    w = WORKLOADS[name]
    inp = make_inputs(w)
    say("workload", name, "full")
    y, ls = _run_fwd(inp)
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True)
    tol = TOL[inp["u"].dtype]
    e_y = rel_err(to_np(y), yr)
    del yr
    e_s = rel_err(to_np(ls), lsr)
    say(f"  {name}: y err {e_y:.3e}, last_state err {e_s:.3e} (bound {tol})")
    assert e_y <= tol, f"{name} y err {e_y:.3e}"
    assert e_s <= max(tol, 1e-5), f"{name} last_state err {e_s:.3e}"


def test_shard_shapes():
    """One GPU's share of an 8-way channel split (D / 8) of the 2.8B forward
    and of the backward workload, in the schedule the bench's shard leg times:
    every output against the float64 oracle."""
    w = WORKLOADS["m2p8b_d8"]
    inp = make_inputs(w)
    say("workload m2p8b_d8")
    y, ls = _run_fwd(inp)
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True)
    tol = TOL[inp["u"].dtype]
    assert rel_err(to_np(y), yr) <= tol
    assert rel_err(to_np(ls), lsr) <= max(tol, 1e-5)
    say("workload bwd_d8")
    errs = _check_bwd(make_inputs(WORKLOADS["bwd_d8"]), label="bwd_d8 workload")
    say("bwd_d8 errors", errs)


def test_fwd_deterministic():
    w = WORKLOADS["m2p8b"]
    inp = to_dev(make_inputs(w))
    args = [inp[k] for k in KEYS]
    y1, _ = ss.fwd(*args)
    y2, _ = ss.fwd(*args)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y3, _ = ss.fwd(*args)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    inp = to_dev(make_inputs(WORKLOADS["m130m"]))
    args = [inp[k] for k in KEYS]
    a, la = ss.fwd(*args, return_last_state=True)
    b, lb = ss.fwd(*args, return_last_state=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_native_library_is_loaded():
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert os.path.realpath(ss.library_path) in maps


# ----------------------------------------------------------------- backward

def _check_bwd(inp, sp=True, chunk_len=0, label=""):
    say("bwd", label, tuple(inp["u"].shape), inp["A"].shape[1], inp["u"].dtype)
    d = to_dev(inp)
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], delta_softplus=sp, chunk_len=chunk_len)
    torch.cuda.synchronize()
    r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], delta_softplus=sp)
    tol = TOL[inp["u"].dtype]
    errs = {}
    for k in GRADS:
        if r[k] is None:
            assert g[k] is None
            continue
        errs[k] = rel_err(to_np(g[k]), r[k])
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, f"{label}: {bad} (tol {tol})"
    return errs


BWD_SHAPES = [(1, 1, 1, 1), (1, 5, 3, 4), (2, 16, 64, 16), (2, 17, 65, 16), (1, 100, 300, 16),
              (3, 63, 31, 8), (1, 47, 20, 17), (1, 33, 10, 64), (1, 20, 9, 130), (1, 18, 5, 256),
              (2, 300, 257, 16), (2, 2048, 512, 16),
              # 4 states per lane (N = 17 .. 32): 32-step chunks, ragged tails, padded states
              (2, 300, 72, 32), (1, 129, 40, 24), (2, 2048, 512, 32)]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes_f32(shape):
    Bn, L, D, N = shape
    _check_bwd(random_inputs(Bn, L, D, N, seed=600 + sum(shape), backward=True),
               label=str(shape))


@pytest.mark.parametrize("combo", range(16))
def test_bwd_optional_combinations(combo):
    has_D, has_z, has_bias, sp = [bool(combo >> i & 1) for i in range(4)]
    inp = random_inputs(2, 70, 40, 16, seed=700 + combo, has_D=has_D, has_z=has_z,
                        has_bias=has_bias, backward=True)
    if not sp:
        inp["delta"] = inp["delta"].abs() * 0.3
        if inp["delta_bias"] is not None:
            inp["delta_bias"] = inp["delta_bias"].abs() * 0.01
    for chunk in (0, 5):
        _check_bwd(inp, sp=sp, chunk_len=chunk, label=f"combo{combo}/chunk{chunk}")


@pytest.mark.parametrize("io,pa", [("bf16", "f32"), ("f16", "f32"), ("bf16", "bf16")])
def test_bwd_half_dtypes(io, pa):
    inp = random_inputs(2, 90, 70, 16, seed=800, io_dtype=io, param_dtype=pa, backward=True)
    _check_bwd(inp, label=f"{io}/{pa}")


def test_bwd_degenerate():
    inp = random_inputs(2, 30, 20, 1, seed=901, backward=True)
    inp["A"], inp["B"], inp["C"] = inp["A"][:, :0], inp["B"][:, :, :0], inp["C"][:, :, :0]
    _check_bwd(inp, label="N0")
    # L = 0: every reduced gradient is an empty sum
    inp = random_inputs(2, 1, 20, 4, seed=902, backward=True)
    for k in ("u", "delta", "z", "B", "C", "dy"):
        inp[k] = inp[k][:, :0].contiguous()
    d = to_dev(inp)
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"])
    torch.cuda.synchronize()
    for k in ("dA", "dD", "ddelta_bias"):
        assert torch.all(g[k] == 0), k


def test_bwd_workload():
    w = WORKLOADS["bwd"]
    inp = make_inputs(w)
    errs = _check_bwd(inp, label="bwd workload")
    say("bwd workload errors", errs)


def test_bwd_deterministic():
    inp = to_dev(make_inputs(WORKLOADS["bwd"]))
    args = [inp[k] for k in KEYS]
    g1 = ss.bwd(*args, dy=inp["dy"])
    g2 = ss.bwd(*args, dy=inp["dy"])
    torch.cuda.synchronize()
    for k in GRADS:
        assert torch.equal(g1[k], g2[k]), k


def test_autograd_function():
    inp = random_inputs(2, 40, 24, 16, seed=950, backward=True)
    d = to_dev(inp)
    leaves = {k: (None if d[k] is None else d[k].clone().requires_grad_(True)) for k in KEYS}
    y = ss.selective_scan(*[leaves[k] for k in KEYS])
    y.backward(d["dy"])
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"])
    for k, gk in zip(KEYS, GRADS):
        assert torch.equal(leaves[k].grad, g[gk]), k


# ------------------------------------------------------------- initial state

def _state(inp, seed, scale=1.0):
    """A seeded initial state [B, D, N] in the parameter dtype."""
    Bn, L, D = inp["u"].shape
    N = inp["A"].shape[1]
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(Bn, D, N, generator=g, dtype=torch.float64) * scale).to(inp["A"].dtype)


H0_SHAPES = [((2, 150, 72, 16), "f32"), ((2, 100, 65, 16), "f32"), ((1, 60, 20, 64), "f32"),
             ((1, 40, 9, 130), "f32"), ((2, 90, 72, 8), "bf16"), ((2, 70, 40, 32), "f16"),
             ((1, 1, 33, 16), "f32")]


@pytest.mark.parametrize("shape,io", H0_SHAPES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_fwd_h0(shape, io):
    inp = random_inputs(*shape, seed=1200 + sum(shape), io_dtype=io)
    h0 = _state(inp, 1300 + shape[2])
    d = to_dev(inp)
    for chunk in (0, 24):
        say("fwd h0", shape, io, "chunk", chunk)
        y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True, chunk_len=chunk,
                       h0=h0.to(DEV))
        torch.cuda.synchronize()
        yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
        tol = TOL[inp["u"].dtype]
        assert rel_err(to_np(y), yr) <= tol, f"y chunk {chunk}"
        assert rel_err(to_np(ls), lsr) <= max(tol, TOL[inp["A"].dtype]), f"state chunk {chunk}"


def test_fwd_h0_split_sequence_and_empty():
    inp = random_inputs(2, 300, 96, 16, seed=1401)
    h0 = _state(inp, 1402).to(DEV)
    d = to_dev(inp)
    args = [d[k] for k in KEYS]
    y, ls = ss.fwd(*args, return_last_state=True, h0=h0)
    cut = lambda t, a, b: t[:, a:b].contiguous() if t is not None and t.dim() == 3 else t
    first = [cut(t, 0, 113) for t in args]
    second = [cut(t, 113, 300) for t in args]
    y1, l1 = ss.fwd(*first, return_last_state=True, h0=h0)
    y2, l2 = ss.fwd(*second, return_last_state=True, h0=l1)
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0.cpu())
    assert rel_err(to_np(torch.cat([y1, y2], 1)), yr) <= 1e-5
    assert rel_err(to_np(l2), lsr) <= 1e-5
    assert rel_err(to_np(y), yr) <= 1e-5
    # L = 0: the final state is h0; in place it stays h0
    e = [cut(t, 0, 0) for t in args]
    _, le = ss.fwd(*e, return_last_state=True, h0=h0)
    st = h0.clone()
    ss.fwd(*e, h0=st, last_state=st)
    torch.cuda.synchronize()
    assert torch.equal(le, h0) and torch.equal(st, h0)


@pytest.mark.parametrize("io,D", [("f32", 64), ("bf16", 72), ("f32", 33)])
def test_decode_step_in_place(io, D):
    """L steps of decode_step on one state equal one call over the sequence."""
    inp = random_inputs(3, 24, D, 16, seed=1500 + D, io_dtype=io)
    h0 = _state(inp, 1501)
    d = to_dev(inp)
    state = h0.to(DEV).clone()
    ys = []
    for t in range(24):
        sl = lambda k: None if d[k] is None else d[k][:, t].contiguous()
        ys.append(ss.decode_step(state, sl("u"), sl("delta"), d["A"], sl("B"), sl("C"), d["D"],
                                 sl("z"), d["delta_bias"]))
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    tol = TOL[inp["u"].dtype]
    assert rel_err(to_np(torch.stack(ys, 1)), yr) <= tol
    assert rel_err(to_np(state), lsr) <= max(tol, 1e-5)


PADDED_CASES = [  # (B, L, D, N, io, R, chunk): N > 64 short of its lanes' states
    (2, 150, 40, 100, "f32", None, 0), (1, 90, 24, 200, "bf16", None, 16),
    (2, 70, 33, 65, "f16", 5, 0), (1, 130, 20, 129, "f32", 3, 24),
]


@pytest.mark.parametrize("case", PADDED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fwd_padded_rows(case):
    """The general forward copies B / C into rows of NS * G elements (zero past
    N) when N falls short of them: against the oracle with h0, strided B / C
    and forced chunks, and equal to the packed call bit for bit."""
    Bn, L, D, N, io, R, chunk = case
    inp = random_inputs(Bn, L, D, N, seed=3400 + N + L, io_dtype=io)
    h0 = _state(inp, 3401 + D)
    d = to_dev(inp)
    args = {k: d[k] for k in KEYS}
    say("padded rows", case)
    y0, l0 = ss.fwd(**args, return_last_state=True, chunk_len=chunk, h0=h0.to(DEV))
    if R is not None:
        _, Bv, Cv = _xdbl(d["B"], d["C"], R, 3402 + R)
        args.update(B=Bv, C=Cv)
    y1, l1 = ss.fwd(**args, return_last_state=True, chunk_len=chunk, h0=h0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(l0, l1)
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    tol = TOL[inp["u"].dtype]
    assert rel_err(to_np(y1), yr) <= tol
    assert rel_err(to_np(l1), lsr) <= max(tol, 1e-5)


SHORT_CASES = [  # (io, param dtype, N, L, R): R = columns before B in an xdbl-like row, or None
    ("bf16", "f32", 16, 7, 5),      # B / C rows not 4-byte aligned: element loads
    ("bf16", "f32", 16, 16, 6),     # strided, 32-bit word loads
    ("f16", "f32", 32, 3, None),    # 8 states per lane
    ("f32", "f32", 8, 12, None),    # 2 states per lane: element loads
    ("bf16", "bf16", 16, 5, None),  # 16-bit parameters
    ("f32", "f32", 16, 1, 3),
]


@pytest.mark.parametrize("case", SHORT_CASES, ids=lambda c: "-".join(map(str, c)))
def test_short_sequence_loads(case):
    """The short-sequence kernel (L <= 16) with its next-step prefetch and the
    B / C word loads on and off, against the oracle, with h0."""
    io, pa, N, L, R = case
    inp = random_inputs(2, L, 72, N, seed=3300 + N + L, io_dtype=io, param_dtype=pa)
    h0 = _state(inp, 3301 + L)
    d = to_dev(inp)
    args = {k: d[k] for k in KEYS}
    if R is not None:
        _, Bv, Cv = _xdbl(d["B"], d["C"], R, 3302 + R)
        args.update(B=Bv, C=Cv)
    say("short sequence", case)
    y, ls = ss.fwd(**args, return_last_state=True, h0=h0.to(DEV))
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    tol = TOL[inp["u"].dtype]
    assert rel_err(to_np(y), yr) <= tol
    assert rel_err(to_np(ls), lsr) <= max(tol, 1e-5)


BWD_H0_SHAPES = [((2, 150, 72, 16), "f32"), ((2, 300, 257, 16), "f32"), ((1, 47, 20, 17), "f32"),
                 ((1, 33, 10, 64), "f32"), ((2, 90, 70, 16), "bf16"), ((1, 1, 9, 16), "f32")]


@pytest.mark.parametrize("shape,io", BWD_H0_SHAPES, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_bwd_h0(shape, io):
    inp = random_inputs(*shape, seed=1600 + sum(shape), io_dtype=io, backward=True)
    h0 = _state(inp, 1700 + shape[2])
    d = to_dev(inp)
    r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
    tol = TOL[inp["u"].dtype]
    for chunk in (0, 24):
        say("bwd h0", shape, io, "chunk", chunk)
        g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
        torch.cuda.synchronize()
        for k in GRADS + ("dh0",):
            if r[k] is None:
                assert g[k] is None
                continue
            e = rel_err(to_np(g[k]), r[k])
            assert e <= tol, f"{k} chunk {chunk}: {e:.3e}"


def test_bwd_h0_empty_and_autograd():
    inp = random_inputs(2, 1, 20, 4, seed=1801, backward=True)
    h0 = _state(inp, 1802).to(DEV)
    for k in ("u", "delta", "z", "B", "C", "dy"):
        inp[k] = inp[k][:, :0].contiguous()
    d = to_dev(inp)
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], h0=h0)
    torch.cuda.synchronize()
    assert torch.all(g["dh0"] == 0)
    inp = random_inputs(2, 40, 24, 16, seed=1803, backward=True)
    d = to_dev(inp)
    h0 = _state(inp, 1804).to(DEV).requires_grad_(True)
    leaves = {k: (None if d[k] is None else d[k].clone().requires_grad_(True)) for k in KEYS}
    y = ss.selective_scan(*[leaves[k] for k in KEYS], h0=h0)
    (y * d["dy"]).sum().backward()
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], h0=h0.detach())
    torch.cuda.synchronize()
    assert torch.equal(h0.grad, g["dh0"])
    assert torch.equal(leaves["A"].grad, g["dA"])


def test_decode_step_2p8b_layer():
    """One in-place step at the 2.8B-shaped layer size (every channel)."""
    w = WORKLOADS["m2p8b"]
    full = make_inputs(w)
    inp = {k: (None if v is None else (v[:, :1].contiguous() if v.dim() == 3 else v))
           for k, v in full.items()}
    h0 = _state(inp, 1901)
    d = to_dev(inp)
    state = h0.to(DEV).clone()
    y, _ = ss.fwd(*[d[k] for k in KEYS], h0=state, last_state=state)
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    assert rel_err(to_np(y), yr) <= TOL[inp["u"].dtype]
    assert rel_err(to_np(state), lsr) <= 1e-5


@pytest.mark.parametrize("L", [1, 2, 7, 16])
@pytest.mark.parametrize("N,io", [(4, "f32"), (16, "f32"), (16, "bf16"), (32, "f16"), (9, "bf16")])
def test_fwd_short_sequences(L, N, io):
    """Sequences of at most 16 steps run one lane per channel (decode steps)."""
    inp = random_inputs(3, L, 300, N, seed=2000 + 37 * L + N, io_dtype=io)
    for with_h0 in (False, True):
        h0 = _state(inp, 2100 + L) if with_h0 else None
        d = to_dev(inp)
        y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True,
                       h0=None if h0 is None else h0.to(DEV))
        torch.cuda.synchronize()
        yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
        tol = TOL[inp["u"].dtype]
        assert rel_err(to_np(y), yr) <= tol
        assert rel_err(to_np(ls), lsr) <= max(tol, TOL[inp["A"].dtype])


# ------------------------------------------------------- packed sequences

def _packed(S, lens, D, N, seed, io="f32", backward=False):
    """Packed inputs for sequences of the given lengths (rows of one long
    seeded batch), their int32 offsets and the longest length."""
    T = int(sum(lens))
    inp = random_inputs(1, max(T, 1), D, N, seed=seed, io_dtype=io, backward=backward)
    p = {k: (None if v is None else (v[0, :T].contiguous() if v.dim() == 3 else v))
         for k, v in inp.items()}
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return p, cu, int(max(lens)) if len(lens) else 0


VARLEN_CASES = [([37, 0, 130, 5, 64], 72, 16, "f32"), ([300, 1, 77], 96, 16, "bf16"),
                ([9, 16, 3, 12], 40, 16, "f32"), ([50, 200], 20, 64, "f32"),
                ([129, 64, 1000], 65, 8, "f16"), ([2048] * 2 + [100], 128, 16, "bf16")]


@pytest.mark.parametrize("lens,D,N,io", VARLEN_CASES, ids=lambda v: str(v))
def test_fwd_varlen(lens, D, N, io):
    p, cu, Lmax = _packed(len(lens), lens, D, N, seed=2200 + sum(lens) % 97, io=io)
    S = len(lens)
    g = torch.Generator().manual_seed(2300 + S)
    h0 = torch.randn(S, D, N, generator=g, dtype=torch.float64).to(p["A"].dtype)
    d = to_dev(p)
    cu_d = torch.as_tensor(cu, device=DEV)
    for chunk in (0, 24):
        for with_h0 in (False, True):
            say("fwd varlen", lens, D, N, io, "chunk", chunk, "h0", with_h0)
            y, ls = ss.fwd_varlen(d["u"], d["delta"], d["A"], d["B"], d["C"], cu_d, Lmax,
                                  d["D"], d["z"], d["delta_bias"], chunk_len=chunk,
                                  h0=h0.to(DEV) if with_h0 else None, return_last_state=True)
            torch.cuda.synchronize()
            yr, lsr = oracle.fwd_varlen(**{k: p[k] for k in KEYS}, cu_seqlens=cu,
                                        h0=h0 if with_h0 else None)
            tol = TOL[p["u"].dtype]
            assert rel_err(to_np(y), yr) <= tol
            assert rel_err(to_np(ls), lsr) <= max(tol, TOL[p["A"].dtype])


@pytest.mark.parametrize("lens,D,N,io", VARLEN_CASES, ids=lambda v: str(v))
def test_bwd_varlen(lens, D, N, io):
    p, cu, Lmax = _packed(len(lens), lens, D, N, seed=2400 + sum(lens) % 89, io=io,
                          backward=True)
    S = len(lens)
    g = torch.Generator().manual_seed(2500 + S)
    h0 = torch.randn(S, D, N, generator=g, dtype=torch.float64).to(p["A"].dtype)
    d = to_dev(p)
    cu_d = torch.as_tensor(cu, device=DEV)
    tol = TOL[p["u"].dtype]
    for with_h0 in (False, True):
        r = oracle.bwd_varlen(**{k: p[k] for k in KEYS}, dy=p["dy"], cu_seqlens=cu,
                              h0=h0 if with_h0 else None)
        for chunk in (0, 24):
            say("bwd varlen", lens, D, N, io, "chunk", chunk, "h0", with_h0)
            gr = ss.bwd_varlen(d["u"], d["delta"], d["A"], d["B"], d["C"], cu_d, Lmax, d["D"],
                               d["z"], d["delta_bias"], d["dy"], chunk_len=chunk,
                               h0=h0.to(DEV) if with_h0 else None)
            torch.cuda.synchronize()
            for k in GRADS + ("dh0",):
                if r[k] is None:
                    assert gr[k] is None
                    continue
                e = rel_err(to_np(gr[k]), r[k])
                assert e <= tol, f"{k} chunk {chunk} h0 {with_h0}: {e:.3e}"


def test_varlen_matches_dense_batch():
    """Equal lengths packed back to back give the dense batch's results bit
    for bit (same kernels, same chunking)."""
    inp = random_inputs(3, 150, 72, 16, seed=2601, backward=True)
    d = to_dev(inp)
    pk = {k: (None if v is None else (v.reshape(-1, v.shape[-1]) if v.dim() == 3 else v))
          for k, v in d.items()}
    cu = torch.arange(0, 451, 150, dtype=torch.int32, device=DEV)
    y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True)
    yv, lsv = ss.fwd_varlen(pk["u"], pk["delta"], pk["A"], pk["B"], pk["C"], cu, 150, pk["D"],
                            pk["z"], pk["delta_bias"], return_last_state=True)
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"])
    gv = ss.bwd_varlen(pk["u"], pk["delta"], pk["A"], pk["B"], pk["C"], cu, 150, pk["D"],
                       pk["z"], pk["delta_bias"], pk["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(-1, 72), yv) and torch.equal(ls, lsv)
    for k in GRADS:
        if g[k] is None:
            continue
        a = g[k].reshape(gv[k].shape)
        assert torch.equal(a, gv[k]), k


# ---------------------------------------------- B / C as strided column slices

@pytest.mark.parametrize("seed", range(16))
def test_varlen_random(seed):
    """Seeded random packed-sequence cases (1-6 sequences of 0-500 steps,
    dtypes, N, forced chunk lengths, h0): forward and backward against the
    oracle."""
    rng = np.random.default_rng(8000 + seed)
    S = int(rng.integers(1, 7))
    lens = [int(rng.choice([0, 1, 2, 15, 16, 17, 63, 64, 65, 130, 257, 500])) for _ in range(S)]
    if sum(lens) == 0:
        lens[0] = 5
    D = int(rng.integers(1, 130))
    N = int(rng.choice([1, 4, 8, 16, 16, 17, 32, 64]))
    io = str(rng.choice(["f32", "f32", "bf16", "f16"]))
    chunk = int(rng.choice([0, 0, 3, 24, 64]))
    with_h0 = bool(rng.random() < 0.5)
    say("varlen random case", seed, lens, D, N, io, "chunk", chunk, "h0", with_h0)
    p, cu, Lmax = _packed(S, lens, D, N, seed=8100 + seed, io=io, backward=True)
    g = torch.Generator().manual_seed(8200 + seed)
    h0 = (torch.randn(S, D, N, generator=g, dtype=torch.float64).to(p["A"].dtype)
          if with_h0 else None)
    d = to_dev(p)
    cu_d = torch.as_tensor(cu, device=DEV)
    hd = None if h0 is None else h0.to(DEV)
    y, ls = ss.fwd_varlen(d["u"], d["delta"], d["A"], d["B"], d["C"], cu_d, Lmax, d["D"],
                          d["z"], d["delta_bias"], chunk_len=chunk, h0=hd, return_last_state=True)
    gr = ss.bwd_varlen(d["u"], d["delta"], d["A"], d["B"], d["C"], cu_d, Lmax, d["D"], d["z"],
                       d["delta_bias"], d["dy"], chunk_len=chunk, h0=hd)
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd_varlen(**{k: p[k] for k in KEYS}, cu_seqlens=cu, h0=h0)
    r = oracle.bwd_varlen(**{k: p[k] for k in KEYS}, dy=p["dy"], cu_seqlens=cu, h0=h0)
    tol = TOL[p["u"].dtype]
    ptol = max(tol, TOL[p["A"].dtype])
    assert rel_err(to_np(y), yr) <= tol
    assert rel_err(to_np(ls), lsr) <= ptol
    for k in GRADS + ("dh0",):
        if r[k] is None:
            assert gr[k] is None
            continue
        e = rel_err(to_np(gr[k]), r[k])
        assert e <= (ptol if k in ("dA", "dD", "ddelta_bias", "dh0") else tol), f"{k}: {e:.3e}"


def _xdbl(B, C, R, seed):
    """A [..., R + 2N] x-projection-like matrix with B at column R and C at
    R + N (the dt columns hold seeded noise), on the device."""
    N = B.shape[-1]
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*B.shape[:-1], R + 2 * N, generator=g, dtype=torch.float64)
    x = x.to(dtype=B.dtype, device=DEV)
    x[..., R:R + N] = B
    x[..., R + N:] = C
    return x, x[..., R:R + N], x[..., R + N:]


STRIDED_CASES = [  # (B, L, D, N, io, R): R = columns before B in each row
    (2, 150, 72, 16, "f32", 5), (2, 300, 96, 16, "bf16", 160), (1, 77, 40, 32, "f16", 7),
    (2, 50, 20, 64, "bf16", 4), (1, 33, 10, 128, "f32", 3), (3, 9, 300, 16, "bf16", 160),
    (1, 2048, 64, 8, "f32", 2),
]


@pytest.mark.parametrize("seed", range(16))
def test_strided_random(seed):
    """Seeded random shapes, dtypes, column offsets R and chunk lengths: B / C
    read as column slices of an x-projection-like matrix give the packed
    call's results bit for bit (forward and backward), dB / dC land in their
    columns, and the other columns stay untouched."""
    rng = np.random.default_rng(9000 + seed)
    Bn = int(rng.integers(1, 4))
    L = int(rng.choice([1, 5, 17, 64, 65, 200, 700]))
    D = int(rng.integers(1, 300))
    N = int(rng.choice([1, 4, 8, 16, 16, 17, 32, 64, 128]))
    io = str(rng.choice(["f32", "bf16", "bf16", "f16"]))
    R = int(rng.choice([1, 2, 3, 4, 7, 8, 160]))
    chunk = int(rng.choice([0, 0, 3, 24]))
    say("strided random case", seed, (Bn, L, D, N), io, "R", R, "chunk", chunk)
    inp = random_inputs(Bn, L, D, N, seed=9100 + seed, io_dtype=io, backward=True)
    h0 = _state(inp, 9200 + seed).to(DEV)
    d = to_dev(inp)
    x, Bv, Cv = _xdbl(d["B"], d["C"], R, 9300 + seed)
    args = {k: d[k] for k in KEYS}
    y0, ls0 = ss.fwd(**args, return_last_state=True, chunk_len=chunk, h0=h0)
    g0 = ss.bwd(**args, dy=d["dy"], chunk_len=chunk, h0=h0)
    args.update(B=Bv, C=Cv)
    y1, ls1 = ss.fwd(**args, return_last_state=True, chunk_len=chunk, h0=h0)
    dx = torch.full_like(x, 7.0)
    g1 = ss.bwd(**args, dy=d["dy"], chunk_len=chunk, h0=h0, dB=dx[..., R:R + N],
                dC=dx[..., R + N:])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(ls0, ls1)
    assert torch.all(dx[..., :R] == 7.0)
    for k in GRADS + ("dh0",):
        if g0[k] is not None:
            assert torch.equal(g0[k], g1[k]), k


@pytest.mark.parametrize("case", STRIDED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fwd_strided_bc(case):
    Bn, L, D, N, io, R = case
    inp = random_inputs(Bn, L, D, N, seed=2700 + L + N, io_dtype=io)
    h0 = _state(inp, 2701 + D)
    d = to_dev(inp)
    x, Bv, Cv = _xdbl(d["B"], d["C"], R, 2702 + R)
    assert not Bv.is_contiguous()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    tol = TOL[inp["u"].dtype]
    for chunk in (0, 24):
        say("fwd strided", case, "chunk", chunk)
        args = {k: d[k] for k in KEYS}
        y0, ls0 = ss.fwd(**args, return_last_state=True, chunk_len=chunk, h0=h0.to(DEV))
        args.update(B=Bv, C=Cv)
        y1, ls1 = ss.fwd(**args, return_last_state=True, chunk_len=chunk, h0=h0.to(DEV))
        torch.cuda.synchronize()
        assert rel_err(to_np(y1), yr) <= tol
        assert rel_err(to_np(ls1), lsr) <= max(tol, TOL[inp["A"].dtype])
        # the same kernels on the same values: identical to the packed call
        # (16-byte row alignment decides between two bit-identical kernels)
        assert torch.equal(y0, y1) and torch.equal(ls0, ls1)


@pytest.mark.parametrize("case", STRIDED_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_strided_bc(case):
    Bn, L, D, N, io, R = case
    inp = random_inputs(Bn, L, D, N, seed=2800 + L + N, io_dtype=io, backward=True)
    h0 = _state(inp, 2801 + D)
    d = to_dev(inp)
    x, Bv, Cv = _xdbl(d["B"], d["C"], R, 2802 + R)
    r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
    tol = TOL[inp["u"].dtype]
    for chunk in (0, 5):
        say("bwd strided", case, "chunk", chunk)
        args = {k: d[k] for k in KEYS}
        g0 = ss.bwd(**args, dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
        # dB / dC straight into the matching columns of a d_xdbl buffer whose
        # other columns hold a sentinel that must survive
        dx = torch.full_like(x, 7.0)
        args.update(B=Bv, C=Cv)
        g1 = ss.bwd(**args, dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV),
                    dB=dx[..., R:R + N], dC=dx[..., R + N:])
        torch.cuda.synchronize()
        assert torch.all(dx[..., :R] == 7.0)
        assert torch.equal(dx[..., R:R + N], g0["dB"]) and torch.equal(dx[..., R + N:], g0["dC"])
        for k in GRADS + ("dh0",):
            if r[k] is None:
                continue
            assert torch.equal(g0[k], g1[k]), k
            e = rel_err(to_np(g1[k]), r[k])
            assert e <= tol, f"{k} chunk {chunk}: {e:.3e}"
        # freshly allocated strided outputs keep B's layout
        g2 = ss.bwd(**args, dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
        torch.cuda.synchronize()
        assert g2["dB"].stride() == Bv.stride() and torch.equal(g2["dB"], g0["dB"])


@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 8])
def test_bwd_long_memory_short_chunks(chunk):
    """f32, L = 2048 with an initial state and slowly decaying states, cut into
    very short chunks: every chunk boundary passes the states through the
    carry's closed-form decay, so errors there add up along the sequence (dz,
    an ill-conditioned readout here, is where it shows first: the sequential
    f32 loop itself reaches 2.4e-5 on it, and 1.75e-5 on y).  The carries
    fold their chains in double and round each carried state once, so every
    output stays within the f32 bound at every chunk length, 1-step chunks
    (every state through the carry) included."""
    inp = random_inputs(1, 2048, 64, 8, seed=2800 + 2048 + 8, backward=True)
    h0 = _state(inp, 2801 + 64)
    d = to_dev(inp)
    say("bwd long memory", "chunk", chunk)
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
    y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True, chunk_len=chunk,
                   h0=h0.to(DEV))
    torch.cuda.synchronize()
    r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
    errs = {k: rel_err(to_np(g[k]), r[k]) for k in GRADS + ("dh0",) if r[k] is not None}
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    errs["last_state"] = rel_err(to_np(ls), lsr)
    errs["y"] = rel_err(to_np(y), yr)
    say("  ", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= 1e-5}
    assert not bad, bad


@pytest.mark.parametrize("records", [16, 17, 32, 33, 64, 65, 128, 129, 300])
def test_carry_chain_lengths(records):
    """The chunk carries split a chain of M = K - 1 records over 1, 4 or 8
    lanes (one lane up to 32 records, in rounds of 16; 4 lanes up to 64; 8
    above, in rounds of 128 records past that): M at each boundary, forward
    and backward, with h0 and a channel count that leaves part of the last
    block of chains empty."""
    chunk = 4
    inp = random_inputs(2, chunk * (records + 1) - 1, 48, 16, seed=3100 + records,
                        backward=True)
    h0 = _state(inp, 3200 + records)
    d = to_dev(inp)
    say("carry chain", records, "records", tuple(inp["u"].shape))
    y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True, chunk_len=chunk,
                   h0=h0.to(DEV))
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
    errs = {"y": rel_err(to_np(y), yr), "last_state": rel_err(to_np(ls), lsr)}
    errs.update({k: rel_err(to_np(g[k]), r[k]) for k in GRADS + ("dh0",) if r[k] is not None})
    say("  ", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= 1e-5}
    assert not bad, bad


def test_strided_bc_varlen_and_empty():
    lens = [37, 0, 130, 5, 64]
    D, N, R = 72, 16, 6
    p, cu, Lmax = _packed(len(lens), lens, D, N, seed=2901, backward=True)
    d = to_dev(p)
    cu_d = torch.as_tensor(cu, device=DEV)
    x, Bv, Cv = _xdbl(d["B"], d["C"], R, 2902)
    yr, lsr = oracle.fwd_varlen(**{k: p[k] for k in KEYS}, cu_seqlens=cu)
    r = oracle.bwd_varlen(**{k: p[k] for k in KEYS}, dy=p["dy"], cu_seqlens=cu)
    args = {k: d[k] for k in KEYS if k not in ("B", "C")}
    y, ls = ss.fwd_varlen(B=Bv, C=Cv, cu_seqlens=cu_d, max_seqlen=Lmax, return_last_state=True,
                          **args)
    dx = torch.full_like(x, -3.0)
    g = ss.bwd_varlen(B=Bv, C=Cv, cu_seqlens=cu_d, max_seqlen=Lmax, dy=d["dy"],
                      dB=dx[:, R:R + N], dC=dx[:, R + N:], **args)
    torch.cuda.synchronize()
    assert rel_err(to_np(y), yr) <= 1e-5 and rel_err(to_np(ls), lsr) <= 1e-5
    for k in GRADS:
        if r[k] is not None:
            assert rel_err(to_np(g[k]), r[k]) <= 1e-5, k
    assert torch.all(dx[:, :R] == -3.0)
    # D = 0: no terms reach dB / dC, which are zeroed row by row in place
    inp = random_inputs(2, 20, 1, 4, seed=2903, backward=True)
    for k in ("u", "delta", "z", "dy"):
        inp[k] = inp[k][..., :0].contiguous()
    for k in ("A", "D", "delta_bias"):
        inp[k] = inp[k][:0].contiguous()
    d = to_dev(inp)
    x, Bv, Cv = _xdbl(d["B"], d["C"], 3, 2904)
    dx = torch.full_like(x, 5.0)
    args = {k: d[k] for k in KEYS}
    args.update(B=Bv, C=Cv)
    ss.bwd(**args, dy=d["dy"], dB=dx[..., 3:7], dC=dx[..., 7:])
    torch.cuda.synchronize()
    assert torch.all(dx[..., :3] == 5.0) and torch.all(dx[..., 3:] == 0)


# ------------------------------------------------------- complex A / B / C

def _complex_inputs(Bn, L, D, N, seed, io="f32", pa="f32", backward=False):
    """Real tensors from the seeded recipe plus complex A, B, C and h0 as
    (re, im) pairs: Re A = -exp(N(0,1)), Im A = N(0, 2); B, C, h0 ~ N(0, 1)."""
    inp = random_inputs(Bn, L, D, max(N, 1), seed=seed, io_dtype=io, param_dtype=pa,
                        backward=backward)
    g = torch.Generator().manual_seed(seed + 7)
    iod, pad = inp["u"].dtype, inp["D"].dtype
    A = torch.stack([-torch.exp(torch.randn(D, N, generator=g, dtype=torch.float64)),
                     2.0 * torch.randn(D, N, generator=g, dtype=torch.float64)], -1)
    inp["A"] = A.to(pad)
    inp["B"] = torch.randn(Bn, L, N, 2, generator=g, dtype=torch.float64).to(iod)
    inp["C"] = torch.randn(Bn, L, N, 2, generator=g, dtype=torch.float64).to(iod)
    h0 = torch.randn(Bn, D, N, 2, generator=g, dtype=torch.float64).to(pad)
    return inp, h0


COMPLEX_CASES = [  # (B, L, D, N, io): N covers every lanes-per-channel bucket
    (2, 70, 40, 1, "f32"), (2, 150, 72, 4, "f32"), (1, 300, 65, 16, "f32"),
    (2, 90, 33, 17, "f32"), (1, 64, 20, 64, "f32"), (1, 40, 9, 130, "f32"),
    (1, 33, 7, 256, "f32"), (2, 120, 96, 16, "bf16"), (1, 77, 40, 8, "f16"),
    (1, 2048, 32, 16, "f32"),
    # one lane per (channel, state) with idle lanes (N = 12), a tail channel
    # block (D = 33) and partial 16-step tiles (L = 77)
    (2, 77, 33, 12, "f16"), (1, 77, 33, 12, "f32"),
]


@pytest.mark.parametrize("case", COMPLEX_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fwd_complex(case):
    Bn, L, D, N, io = case
    inp, h0 = _complex_inputs(Bn, L, D, N, seed=3000 + L + N, io=io)
    d = to_dev(inp)
    tol = TOL[inp["u"].dtype]
    for with_h0 in (False, True):
        hh = h0 if with_h0 else None
        yr, lsr = oracle.fwd_complex(**{k: inp[k] for k in KEYS}, h0=hh)
        for chunk in (0, 24):
            say("fwd complex", case, "chunk", chunk, "h0", with_h0)
            y, ls = ss.fwd_complex(*[d[k] for k in KEYS], h0=None if hh is None else hh.to(DEV),
                                   return_last_state=True, chunk_len=chunk)
            torch.cuda.synchronize()
            assert rel_err(to_np(y), yr) <= tol, f"y chunk {chunk}"
            assert rel_err(to_np(ls), lsr) <= max(tol, TOL[inp["A"].dtype]), f"ls chunk {chunk}"


@pytest.mark.parametrize("case", COMPLEX_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_complex(case):
    Bn, L, D, N, io = case
    inp, h0 = _complex_inputs(Bn, L, D, N, seed=3100 + L + N, io=io, backward=True)
    d = to_dev(inp)
    tol = TOL[inp["u"].dtype]
    for with_h0 in (False, True):
        hh = h0 if with_h0 else None
        r = oracle.bwd_complex(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=hh)
        for chunk in (0, 3):
            say("bwd complex", case, "chunk", chunk, "h0", with_h0)
            g = ss.bwd_complex(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk,
                               h0=None if hh is None else hh.to(DEV))
            torch.cuda.synchronize()
            for k in GRADS + ("dh0",):
                if r[k] is None:
                    assert g[k] is None
                    continue
                e = rel_err(to_np(g[k]), r[k])
                assert e <= tol, f"{k} chunk {chunk} h0 {with_h0}: {e:.3e}"


@pytest.mark.parametrize("seed", range(24))
def test_complex_random_shapes(seed):
    """Seeded random complex cases (every lanes-per-channel bucket up to
    N = 256, io dtypes, forced chunk lengths, h0): forward and backward
    against the oracle."""
    rng = np.random.default_rng(7000 + seed)
    N = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 17, 24, 32, 40, 64, 65, 100, 128, 200, 256]))
    L = int(rng.choice([1, 2, 7, 33, 64, 65, 130, 300]))
    D = int(rng.integers(1, 130))
    Bn = int(rng.integers(1, 4))
    io = str(rng.choice(["f32", "f32", "bf16", "f16"]))
    chunk = int(rng.choice([0, 0, 3, 8, 24]))
    with_h0 = bool(rng.random() < 0.5)
    say("complex random case", seed, (Bn, L, D, N), io, "chunk", chunk, "h0", with_h0)
    inp, h0 = _complex_inputs(Bn, L, D, N, seed=7100 + seed, io=io, backward=True)
    hh = h0 if with_h0 else None
    d = to_dev(inp)
    hd = None if hh is None else hh.to(DEV)
    y, ls = ss.fwd_complex(*[d[k] for k in KEYS], h0=hd, return_last_state=True, chunk_len=chunk)
    g = ss.bwd_complex(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=hd)
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd_complex(**{k: inp[k] for k in KEYS}, h0=hh)
    r = oracle.bwd_complex(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=hh)
    tol = TOL[inp["u"].dtype]
    assert rel_err(to_np(y), yr) <= tol
    assert rel_err(to_np(ls), lsr) <= max(tol, TOL[inp["A"].dtype])
    for k in GRADS + ("dh0",):
        if r[k] is None:
            assert g[k] is None
            continue
        e = rel_err(to_np(g[k]), r[k])
        assert e <= tol, f"{k}: {e:.3e}"


@pytest.mark.parametrize("chunk", [0, 1, 5, 16, 17])
def test_complex_lanes_edges(chunk):
    """The lane-per-state kernels (8 < N <= 16 forward, N <= 16 backward) on
    a single partial channel block (D = 5), N = 9 (7 idle lanes per row),
    sequences of 19 steps (a partial 16-step tile) and forced chunks of 1 to
    17 steps, with h0: forward and backward against the oracle."""
    Bn, L, D, N = 3, 19, 5, 9
    inp, h0 = _complex_inputs(Bn, L, D, N, seed=7301 + chunk, backward=True)
    d = to_dev(inp)
    say("complex lanes edges, chunk", chunk)
    y, ls = ss.fwd_complex(*[d[k] for k in KEYS], h0=h0.to(DEV), return_last_state=True,
                           chunk_len=chunk)
    g = ss.bwd_complex(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=h0.to(DEV))
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd_complex(**{k: inp[k] for k in KEYS}, h0=h0)
    r = oracle.bwd_complex(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
    assert rel_err(to_np(y), yr) <= 1e-5
    assert rel_err(to_np(ls), lsr) <= 1e-5
    for k in GRADS + ("dh0",):
        if r[k] is not None:
            e = rel_err(to_np(g[k]), r[k])
            assert e <= 1e-5, f"{k} chunk {chunk}: {e:.3e}"


def test_complex_extreme_inputs():
    """The complex decay's edge branches: dt up to 30 with Im A up to ~1e4
    (angles dt Im A past 4096 take the double-precision reduction), Re A at
    -80 (e^w below the float range: a clamps to 0), and A = 0 on some states:
    forward and backward against the oracle.  dt is taken without softplus,
    so both sides use the same float dt: a float-rounded dt would itself move
    such angles by more than the tolerance (|dt Im A| ~ 1e5 times 6e-8)."""
    Bn, L, D, N = 2, 61, 24, 16
    inp, h0 = _complex_inputs(Bn, L, D, N, seed=5201, backward=True)
    g = torch.Generator().manual_seed(5202)
    pick = torch.randint(0, 5, (Bn, L, D), generator=g)
    vals = torch.tensor([1e-3, 0.3, 2.0, 9.0, 30.0], dtype=torch.float64)
    inp["delta"] = vals[pick].to(inp["delta"].dtype)
    inp["delta_bias"] = torch.zeros_like(inp["delta_bias"])
    A = inp["A"].to(torch.float64).clone()
    A[:, 1::4, 1] *= 3000.0                   # fast rotations
    A[:, 2::4, 0] = -80.0                     # decays past the float range at dt = 30
    A[:, ::4] = 0.0                           # a = 1
    inp["A"] = A.to(inp["A"].dtype)
    d = to_dev(inp)
    for chunk in (0, 8):
        say("complex extreme inputs, chunk", chunk)
        y, ls = ss.fwd_complex(*[d[k] for k in KEYS], delta_softplus=False, h0=h0.to(DEV),
                               return_last_state=True, chunk_len=chunk)
        gr = ss.bwd_complex(*[d[k] for k in KEYS], dy=d["dy"], delta_softplus=False,
                            chunk_len=chunk, h0=h0.to(DEV))
        torch.cuda.synchronize()
        yr, lsr = oracle.fwd_complex(**{k: inp[k] for k in KEYS}, delta_softplus=False, h0=h0)
        r = oracle.bwd_complex(**{k: inp[k] for k in KEYS}, dy=inp["dy"], delta_softplus=False,
                               h0=h0)
        assert rel_err(to_np(y), yr) <= 1e-5
        assert rel_err(to_np(ls), lsr) <= 1e-5
        for k in GRADS + ("dh0",):
            if r[k] is not None:
                e = rel_err(to_np(gr[k]), r[k])
                assert e <= 1e-5, f"{k} chunk {chunk}: {e:.3e}"


def test_complex_decode_empty_and_determinism():
    # an in-place L = 1 step on a carried complex state
    inp, h0 = _complex_inputs(3, 1, 300, 16, seed=3201)
    d = to_dev(inp)
    state = h0.to(DEV).clone()
    y, _ = ss.fwd_complex(*[d[k] for k in KEYS], h0=state, last_state=state)
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd_complex(**{k: inp[k] for k in KEYS}, h0=h0)
    assert rel_err(to_np(y), yr) <= 1e-5 and rel_err(to_np(state), lsr) <= 1e-5
    # L = 0: the final state is h0, every reduced gradient an empty sum
    inp, h0 = _complex_inputs(2, 1, 20, 4, seed=3202, backward=True)
    for k in ("u", "delta", "z", "B", "C", "dy"):
        inp[k] = inp[k][:, :0].contiguous()
    d = to_dev(inp)
    _, ls = ss.fwd_complex(*[d[k] for k in KEYS], h0=h0.to(DEV), return_last_state=True)
    g = ss.bwd_complex(*[d[k] for k in KEYS], dy=d["dy"], h0=h0.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(ls.cpu(), h0)
    for k in ("dA", "dD", "ddelta_bias", "dh0"):
        assert torch.all(g[k] == 0), k
    # bitwise reproducible, torch complex64 inputs accepted
    inp, h0 = _complex_inputs(2, 200, 64, 16, seed=3203, backward=True)
    d = to_dev(inp)
    args = [d[k] for k in KEYS]
    g1 = ss.bwd_complex(*args, dy=d["dy"], h0=h0.to(DEV))
    cargs = [torch.view_as_complex(x.contiguous()) if k in ("A", "B", "C") else x
             for k, x in zip(KEYS, args)]
    g2 = ss.bwd_complex(*cargs, dy=d["dy"], h0=torch.view_as_complex(h0.to(DEV)))
    torch.cuda.synchronize()
    for k in GRADS + ("dh0",):
        assert torch.equal(g1[k], g2[k]), k


# ------------------------------------- the bench's variant legs at full size

def test_bench_strided_and_varlen_legs():
    """The 2.8B-shaped forward with B/C read from xdbl [8, 2048, 192] equals the
    packed call bit for bit; the same rows as 14 packed sequences match the
    oracle on sampled (sequence, channel) pairs."""
    w = WORKLOADS["m2p8b"]
    inp = make_inputs(w)
    d = to_dev(inp)
    say("bench legs: strided")
    y0, _ = ss.fwd(*[d[k] for k in KEYS])
    R, N = 160, w.dstate
    x, Bv, Cv = _xdbl(d["B"], d["C"], R, 3301)
    args = {k: d[k] for k in KEYS}
    args.update(B=Bv, C=Cv)
    y1, _ = ss.fwd(**args)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    del x, Bv, Cv, y1
    say("bench legs: varlen")
    lens = [2048, 1024, 512, 2048, 1024, 512, 2048, 1024, 512, 2048, 1024, 512, 1024, 1024]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pk = {k: (None if d[k] is None else (d[k].reshape(-1, d[k].shape[-1]) if d[k].dim() == 3
                                          else d[k])) for k in KEYS}
    yv, lsv = ss.fwd_varlen(cu_seqlens=torch.as_tensor(cu, device=DEV), max_seqlen=max(lens),
                            return_last_state=True, **pk)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3302)
    hp = {k: (None if inp[k] is None else (inp[k].reshape(-1, inp[k].shape[-1])
                                           if inp[k].dim() == 3 else inp[k])) for k in KEYS}
    for s in (0, 2, 8, 13):
        a, b = int(cu[s]), int(cu[s + 1])
        seg = {k: (None if hp[k] is None else (hp[k][a:b][None] if k in ("u", "delta", "z", "B", "C")
                                               else hp[k])) for k in KEYS}
        cd = np.concatenate([rng.integers(0, w.dim, 16), [0, 63, 64, w.dim - 1]])
        yr, lsr = oracle.fwd_channels(**seg, chan_b=np.zeros_like(cd), chan_d=cd)
        yg = yv[a:b][:, torch.as_tensor(cd)].T                 # [nchan, len]
        assert rel_err(to_np(yg), yr) <= TOL[inp["u"].dtype], s
        assert rel_err(to_np(lsv[s][torch.as_tensor(cd)]), lsr) <= 1e-5, s


def test_bench_complex_leg():
    """The complex leg's shape (2x2048x1024x16, f32, default schedule): the
    whole forward against the oracle, and the backward's per-channel
    gradients on a slice of channels (dB / dC sum over every channel and are
    covered at the smaller sizes)."""
    inp, h0 = _complex_inputs(2, 2048, 1024, 16, seed=3401, backward=True)
    d = to_dev(inp)
    say("bench legs: complex forward")
    y, ls = ss.fwd_complex(*[d[k] for k in KEYS], return_last_state=True)
    g = ss.bwd_complex(*[d[k] for k in KEYS], dy=d["dy"])
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd_complex(**{k: inp[k] for k in KEYS})
    assert rel_err(to_np(y), yr) <= 1e-5 and rel_err(to_np(ls), lsr) <= 1e-5
    say("bench legs: complex backward (channel slice)")
    sl = slice(0, 96)
    sub = {k: (None if inp[k] is None else
               (inp[k][..., sl] if k in ("u", "delta", "z") else
                inp[k][sl] if k in ("A", "D", "delta_bias") else inp[k])) for k in KEYS}
    r = oracle.bwd_complex(**sub, dy=inp["dy"][..., sl])
    for k, gk in (("du", g["du"][..., sl]), ("ddelta", g["ddelta"][..., sl]),
                  ("dz", g["dz"][..., sl]), ("dA", g["dA"][sl]), ("dD", g["dD"][sl]),
                  ("ddelta_bias", g["ddelta_bias"][sl])):
        e = rel_err(to_np(gk), r[k])
        assert e <= 1e-5, f"{k}: {e:.3e}"


def test_graph_capture_replays():
    """Forward, backward and an in-place decode step captured in one HIP graph:
    every replay (with eager work between replays) matches the eager results
    bit for bit (no memsets inside the library's launches)."""
    inp = random_inputs(2, 300, 96, 16, seed=3501, backward=True)
    d = to_dev(inp)
    args = [d[k] for k in KEYS]
    h0 = _state(inp, 3502).to(DEV)
    y_e, _ = ss.fwd(*args, h0=h0)
    g_e = ss.bwd(*args, dy=d["dy"], h0=h0)
    st = h0.clone()
    step = [None if t is None else (t[:, :1].contiguous() if t.dim() == 3 else t) for t in args]
    ss.fwd(*step, h0=st, last_state=st)
    st_e = st.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    state = h0.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ss.fwd(*args, h0=h0)                 # warm-up allocations outside the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            y_g, _ = ss.fwd(*args, h0=h0)
            g_g = ss.bwd(*args, dy=d["dy"], h0=h0)
            ss.fwd(*step, h0=state, last_state=state)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(3):
        say("graph replay", r)
        state.copy_(h0)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e)
        for k in GRADS + ("dh0",):
            if g_e[k] is not None:
                assert torch.equal(g_g[k], g_e[k]), k
        assert torch.equal(state, st_e)
        ss.fwd(*args)                        # eager work between replays
        torch.cuda.synchronize()


def test_graph_capture_replays_complex():
    """The complex forward and backward (lane-per-state kernels, chunked)
    captured in a HIP graph: every replay, with eager work between replays,
    matches the eager results bit for bit."""
    inp, h0 = _complex_inputs(2, 300, 40, 16, seed=3511, backward=True)
    d = to_dev(inp)
    args = [d[k] for k in KEYS]
    hd = h0.to(DEV)
    y_e, ls_e = ss.fwd_complex(*args, h0=hd, return_last_state=True, chunk_len=64)
    g_e = ss.bwd_complex(*args, dy=d["dy"], h0=hd)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ss.fwd_complex(*args, h0=hd, chunk_len=64)   # warm-up allocations outside the graph
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            y_g, ls_g = ss.fwd_complex(*args, h0=hd, return_last_state=True, chunk_len=64)
            g_g = ss.bwd_complex(*args, dy=d["dy"], h0=hd)
    torch.cuda.current_stream().wait_stream(side)
    for r in range(3):
        say("complex graph replay", r)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e) and torch.equal(ls_g, ls_e)
        for k in GRADS + ("dh0",):
            if g_e[k] is not None:
                assert torch.equal(g_g[k], g_e[k]), k
        ss.fwd_complex(*args)                         # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------ seeded random shapes

def _random_case(seed):
    rng = np.random.default_rng(seed)
    Bn = int(rng.integers(1, 4))
    L = int(rng.choice([1, 2, 5, 16, 17, 63, 64, 65, 130, 257, 700]))
    D = int(rng.choice([1, 3, 8, 31, 32, 33, 64, 100, 257]))
    N = int(rng.choice([1, 4, 8, 12, 16, 17, 32, 40, 64, 100]))
    io = str(rng.choice(["f32", "f32", "bf16", "f16"]))
    pa = "f32" if io == "f32" or rng.random() < 0.7 else io
    opts = dict(has_D=bool(rng.random() < 0.8), has_z=bool(rng.random() < 0.8),
                has_bias=bool(rng.random() < 0.8))
    chunk = int(rng.choice([0, 0, 3, 8, 24, 64]))
    return Bn, L, D, N, io, pa, opts, chunk, bool(rng.random() < 0.5)


@pytest.mark.parametrize("seed", range(64))
def test_random_shapes(seed):
    """Seeded random shapes, dtypes, options, forced chunk lengths and initial
    states: forward and backward against the oracle."""
    Bn, L, D, N, io, pa, opts, chunk, with_h0 = _random_case(4000 + seed)
    say("random case", seed, (Bn, L, D, N), io, pa, opts, "chunk", chunk, "h0", with_h0)
    inp = random_inputs(Bn, L, D, N, seed=4100 + seed, io_dtype=io, param_dtype=pa,
                        backward=True, **opts)
    h0 = _state(inp, 4200 + seed) if with_h0 else None
    d = to_dev(inp)
    hd = None if h0 is None else h0.to(DEV)
    y, ls = ss.fwd(*[d[k] for k in KEYS], return_last_state=True, chunk_len=chunk, h0=hd)
    g = ss.bwd(*[d[k] for k in KEYS], dy=d["dy"], chunk_len=chunk, h0=hd)
    torch.cuda.synchronize()
    yr, lsr = oracle.fwd(**{k: inp[k] for k in KEYS}, return_last_state=True, h0=h0)
    r = oracle.bwd(**{k: inp[k] for k in KEYS}, dy=inp["dy"], h0=h0)
    tol = TOL[inp["u"].dtype]
    assert rel_err(to_np(y), yr) <= tol
    assert rel_err(to_np(ls), lsr) <= max(tol, TOL[inp["A"].dtype])
    for k in GRADS + ("dh0",):
        if r[k] is None:
            assert g[k] is None
            continue
        # parameter-dtype gradients are rounded to that dtype
        t = max(tol, TOL[inp["A"].dtype]) if k in ("dA", "dD", "ddelta_bias", "dh0") else tol
        e = rel_err(to_np(g[k]), r[k])
        assert e <= t, f"{k}: {e:.3e}"


# ------------------------------------------- tensors beyond 2^31 bytes

def test_tensors_beyond_2gib():
    """u / delta / z / y of 4.3 GB each (2 x 262144 x 4096 bf16): the chunked
    forward and the backward address them through per-chunk 32-bit ranges on
    64-bit bases.  Checked on sampled channels (generated on the device with
    a seeded generator; the oracle sees the sampled channels' slices)."""
    Bn, L, D, N = 2, 262144, 4096, 16
    g = torch.Generator(device=DEV).manual_seed(5001)
    rn = lambda *sh: torch.randn(*sh, generator=g, device=DEV)
    u = rn(Bn, L, D).to(torch.bfloat16)
    delta = (rn(Bn, L, D) * 0.5 - 1.0).to(torch.bfloat16)
    z = rn(Bn, L, D).to(torch.bfloat16)
    B = rn(Bn, L, N).to(torch.bfloat16)
    C = rn(Bn, L, N).to(torch.bfloat16)
    A = -torch.exp(rn(D, N))
    Dv = rn(D) * 0.1 + 1.0
    bias = rn(D) * 0.1 - 4.0
    assert u.numel() * u.element_size() >= (1 << 32)       # 4 GiB per stream
    say("beyond 2 GiB: forward", (Bn, L, D, N), "plan", ss.plan(ss._desc_for(u, A, True, 0)).n_chunks)
    y, ls = ss.fwd(u, delta, A, B, C, Dv, z, bias, return_last_state=True)
    torch.cuda.synchronize()
    cd = torch.tensor([0, 1, 255, 2048, 3000, D - 1], device=DEV)
    sl = lambda t: t[..., cd].cpu()
    sub = {"u": sl(u), "delta": sl(delta), "A": A[cd].cpu(), "B": B.cpu(), "C": C.cpu(),
           "D": Dv[cd].cpu(), "z": sl(z), "delta_bias": bias[cd].cpu()}
    yr, lsr = oracle.fwd(**sub, return_last_state=True)
    assert rel_err(to_np(sl(y)), yr) <= 2e-2
    assert rel_err(to_np(ls[:, cd].cpu()), lsr) <= 1e-5
    del y
    say("beyond 2 GiB: backward")
    dy = rn(Bn, L, D).to(torch.bfloat16)
    gr = ss.bwd(u, delta, A, B, C, Dv, z, bias, dy=dy)
    torch.cuda.synchronize()
    r = oracle.bwd(**sub, dy=sl(dy))
    for k in ("du", "ddelta", "dz"):
        e = rel_err(to_np(sl(gr[k])), r[k])
        assert e <= 2e-2, f"{k}: {e:.3e}"
    for k in ("dA", "dD", "ddelta_bias"):
        e = rel_err(to_np(gr[k][cd].cpu()), r[k])
        assert e <= 2e-2, f"{k}: {e:.3e}"
        say(f"  {k} {e:.2e}")
