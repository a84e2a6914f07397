"""Benchmark of the selective scan on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]

A step is one ss_fwd call over the Mamba-2.8B-shaped batch (B=8, L=2048,
D=5120, N=16, bf16 u/delta/B/C/z/y, f32 A/D/delta_bias), inputs resident in
HBM.  The value is forward state-updates/s (B*L*D*N per step / step time) at
the median of K steps, each timed by HIP events on the launch stream with L2
and the MALL evicted (a 1 GiB read) before it; back-to-back timings are
reported beside it.
The same line carries the HBM rate of the algorithmic bytes, the roofline of
the scan kernel (bound by the ALU: the update's instruction mix), the
backward (ss_bwd on the B=2, L=2048, D=2048, N=16 f32 workload), the decode
step, the strided, packed-sequence and complex variants, every workload's
timings with its parity against the float64 oracle, and the oracle's rate on
the host cores.  Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector peak (256 CUs x 2.4 GHz x 256 flop/clk)
# Algorithmic flops of one state update: dt*A (1), exp (1), (dt*u)*B (1),
# a*h + x (2), h*C accumulated (2).
FLOPS_PER_UPDATE = 7
# Backward, per state update: the forward recompute (7) plus the adjoint
# g*C + a*dh (2), dB term dh*(dt*u) (1), du term dh*B (2), q = dh*a*h_prev (2),
# ddt term q*A (2), dA term q*dt (2): 18.
FLOPS_PER_UPDATE_BWD = 18
# Complex forward, per complex state update: dt*A (2), exp and sincos (2),
# (a - 1)*h + x + h (8), (dt*u)*B (2), Re(C*h) accumulated (4): 18.
FLOPS_PER_UPDATE_COMPLEX = 18
# Complex backward, per complex state update: the forward recompute (18) plus
# the adjoint lam = g*conj(C) + dh (4), dB = (dt*u)*lam (2), dC = g*conj(h)
# (2), m = conj(a)*lam (6), dw = m*conj(h_prev) (6), Re(conj(A)*dw) (3),
# dA += dt*dw (4), Re(conj(B)*lam) (3): 48.
FLOPS_PER_UPDATE_COMPLEX_BWD = 48
# The scan is bound by VALU issue, not by HBM (profiles/hw_rates_mi355x.txt):
# a state update is 1 transcendental (v_exp_f32) + 4 FP32 operations (dt*A,
# (dt*u)*B, a*h + x, C*h), and on gfx950 the transcendental takes the same
# issue slots as the FP32 operations (no co-issue, measured).
#
# ALU peak of that instruction mix, from the chip's unit counts and clock:
# 256 CUs x 4 SIMDs = 1024 SIMDs at 2.4 GHz; the FP32 vector peak of 157.3
# TFLOP/s is 32 FMA lanes per SIMD per clock, i.e. one 64-lane FP32
# instruction every 2 clocks; transcendentals run at a quarter of that rate,
# 8 clocks.  One update per lane therefore costs a SIMD 4 x 2 + 8 = 16 clocks
# per 64 updates: 1024 x 64 x 2.4e9 / 16 = 9.83e12 updates/s, 68.8 TFLOP/s
# at 7 flops per update.  (The bare update mix, with no other instruction,
# measures 6.6-7.1e12 updates/s on the box: the clock under this load sits
# below 2.4 GHz.)
SIMDS, CLOCK_HZ = 1024, 2.4e9
OP_CLK, TRANS_CLK = 2, 8        # SIMD clocks per 64-lane FP32 / transcendental instruction


def mix_peak_updates(n_trans: int, n_ops: int) -> float:
    """Updates/s at the ALU peak for n_trans + n_ops instructions per update."""
    return SIMDS * 64 * CLOCK_HZ / (n_trans * TRANS_CLK + n_ops * OP_CLK)


# Measured issue cost of the bare update mix (microbenchmark "upd_clust" at 5
# waves/SIMD, the 2.8B-shaped grid): the floor a real kernel can approach.
MEASURED_UPDATE_MIX = 7.15e12


def mix_floor(updates_per_s: float, n_exp: int, n_ops: int) -> dict:
    floor = mix_peak_updates(n_exp, n_ops)
    return {"updates_per_s": floor, "frac": updates_per_s / floor, "exp_per_update": n_exp,
            "ops_per_update": n_ops}


PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mamba_selective_scan_02_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each measured kernel is built from (its counters go stale when any changes).
KERNEL_SOURCES = {
    "fwd_wide_m2p8b": ["ss_fwd_tile.hip", "ss_device.h", "ss_plan.h", "ss_api.cpp"],
    "ss_bwd_bwd": ["ss_bwd.hip", "ss_bwd_tile.hip", "ss_device.h", "ss_plan.h", "ss_api.cpp"],
}


def kernel_sources_sha(tag: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[tag]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(tag: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary
    (profiles/<tag>_pmc.txt), or None if the kernel's sources changed since
    the counters were taken."""
    path = os.path.join(PROFILES, f"{tag}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_sources_sha:\s*(\S+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_sources_sha(tag):
        return None
    return float(m_b.group(1))


def calibration_copy(nbytes: int = 512 << 20, reps: int = 3):
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read for
    it calibrates the counters (rocprofv3 --pmc runs of this script)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def algorithmic_bytes(w) -> int:
    """Every input read once and every output written once."""
    io = 4 if w.io_dtype == "f32" else 2
    pa = 4 if w.param_dtype == "f32" else 2
    B, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    bld = B * L * D
    n_in_bld = 2 + (1 if w.has_z else 0)              # u, delta, z
    n_out_bld = 1                                      # y
    nbytes = (n_in_bld + n_out_bld) * bld * io + 2 * B * L * N * io + D * N * pa
    nbytes += D * pa * ((1 if w.has_D else 0) + (1 if w.has_bias else 0))
    if w.last_state:
        nbytes += B * D * N * pa
    return nbytes


def algorithmic_bytes_bwd(w) -> int:
    io = 4 if w.io_dtype == "f32" else 2
    pa = 4 if w.param_dtype == "f32" else 2
    B, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    bld = B * L * D
    n_in = 3 + (1 if w.has_z else 0)                   # u, delta, dy, z
    n_out = 2 + (1 if w.has_z else 0)                  # du, ddelta, dz
    nbytes = (n_in + n_out) * bld * io + 4 * B * L * N * io + 2 * D * N * pa
    nbytes += 2 * D * pa * ((1 if w.has_D else 0) + (1 if w.has_bias else 0))
    return nbytes


def time_each(fn, reps: int, scratch=None):
    """Per-call durations (ms) of `reps` calls of fn(), each bracketed by its
    own HIP events on the launch stream.  With `scratch` (a 1 GiB device
    buffer) every call is preceded by a read of the whole buffer, which
    evicts L2 and the 256 MB MALL: the call then reads its inputs from HBM."""
    import torch
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    sink = torch.empty(1, dtype=torch.float32, device="cuda") if scratch is not None else None
    for i in range(reps):
        if scratch is not None:
            # A read of the whole buffer evicts L2 and the MALL without leaving
            # dirty lines behind: after a 1 GiB write, the write-back of up to
            # 256 MB of dirty MALL lines lands inside the timed call (measured:
            # the 2.8B forward reads 406 us after a write, 354-369 us after a
            # read, 352-359 us back to back).
            torch.amax(scratch, dim=0, keepdim=True, out=sink)
        ev[i][0].record(stream)
        fn()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_calls(fn, steps: int, warmup: int):
    """Average duration of fn() over `steps` back-to-back calls, from HIP events
    recorded on the stream the kernels are launched on."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, wall


def state_sweep_leg(ss, steps: int) -> dict:
    """Forward and backward over the state count N = 16 ... 256 on one shape
    (B=2, L=2048, D=2048, f32, D skip / z / delta_bias, seeded inputs of the
    usual distributions): per-update cost and its ratio to N = 16, back to
    back after warm-up (each N picks its own kernels: the 8-lane tile kernels
    up to N = 64 forward and 32 backward, the general ones above)."""
    import torch
    from ss_inputs import random_inputs
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")
    Bn, L, D = 2, 2048, 2048
    out = {"workload": f"B={Bn}, L={L}, D={D}, f32 io and parameters, D skip, z, delta_bias, "
                       "each N timed back to back after warm-up",
           "per_n": {}}
    base = None
    for N in (16, 32, 64, 128, 256):
        log(f"state sweep: N = {N}")
        inp = random_inputs(Bn, L, D, N, seed=4000 + N, backward=True)
        d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
        a = [d[k] for k in keys]
        y = torch.empty_like(d["u"])
        fwd_ms, _ = time_calls(lambda: ss.fwd(*a, y=y), steps, 3)
        bwd_ms, _ = time_calls(lambda: ss.bwd(*a, dy=d["dy"]), steps, 3)
        upd = Bn * L * D * N
        row = {"fwd_us": fwd_ms * 1e3, "bwd_us": bwd_ms * 1e3,
               "fwd_ps_per_update": fwd_ms * 1e9 / upd, "bwd_ps_per_update": bwd_ms * 1e9 / upd}
        if base is None:
            base = row
        row["fwd_per_update_vs_n16"] = row["fwd_ps_per_update"] / base["fwd_ps_per_update"]
        row["bwd_per_update_vs_n16"] = row["bwd_ps_per_update"] / base["bwd_ps_per_update"]
        out["per_n"][str(N)] = row
        del d, a, y, inp
    return out


def alu_roofline(updates_per_s: float, flops_per_update: int, mix=None) -> dict:
    """ALU roofline of a leg.  With mix = (transcendentals, FP32 operations)
    per update, the peak is that instruction mix's ALU peak (mix_peak_updates
    x flops per update); without, the FP32 vector peak."""
    achieved = updates_per_s * flops_per_update / 1e12
    peak = (mix_peak_updates(*mix) * flops_per_update / 1e12 if mix is not None
            else FP32_VECTOR_PEAK_TFLOPS)
    r = {"bound": "alu", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
         "frac": achieved / peak, "flops_per_update": flops_per_update,
         "fp32_vector_frac": achieved / FP32_VECTOR_PEAK_TFLOPS}
    if mix is not None:
        r["mix"] = {"transcendentals_per_update": mix[0], "fp32_ops_per_update": mix[1]}
    return r


def cpu_oracle_rate(run, total_channels: int, updates_per_channel: int, budget_s: float,
                    what: str):
    """Rate of an oracle call `run(nchan)` over the first nchan channels,
    grown until it takes ~1 s and then sized to ~budget_s."""
    import oracle
    n = 1
    while True:
        t0 = time.perf_counter()
        run(n)
        dt = time.perf_counter() - t0
        if dt >= 1.0 or n >= total_channels:
            break
        n = min(total_channels, n * 4)
    n = int(min(total_channels, max(1, n * budget_s / max(dt, 1e-9))))
    t0 = time.perf_counter()
    run(n)
    dt = time.perf_counter() - t0
    upd = n * updates_per_channel
    return {"value": upd / dt, "unit": "state-updates/s", "cores": oracle.default_threads(),
            "kind": "oracle", "sample": f"{what}: the first {n} of {total_channels} channels, "
                                        f"{upd:.3e} updates in {dt:.1f} s"}


def cpu_baseline(w, inp, budget_s: float):
    """The oracle (float64 C loop, threaded over channels) on the host cores,
    on a bounded sample of the same workload: the first channels of every
    batch row, all time steps, sized to take about `budget_s` seconds."""
    import numpy as np
    import oracle
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")
    cores = oracle.default_threads()
    Bn, L, D, N = w.batch, w.seqlen, w.dim, w.dstate
    # calibration: grow a probe until it runs for a second, then size the sample
    nd = min(D, max(1, cores // Bn))
    while True:
        cb = np.repeat(np.arange(Bn), nd)
        cd = np.tile(np.arange(nd), Bn)
        t0 = time.perf_counter()
        oracle.fwd_channels(**{k: inp[k] for k in keys}, chan_b=cb, chan_d=cd, nthreads=cores)
        dt = time.perf_counter() - t0
        if dt >= 1.0 or nd >= D:
            break
        nd = min(D, nd * 4)
    per_chan = dt / cb.size
    nd = int(min(D, max(1, budget_s / per_chan / Bn)))
    cb = np.repeat(np.arange(Bn), nd)
    cd = np.tile(np.arange(nd), Bn)
    t0 = time.perf_counter()
    oracle.fwd_channels(**{k: inp[k] for k in keys}, chan_b=cb, chan_d=cd, nthreads=cores)
    dt = time.perf_counter() - t0
    updates = cb.size * L * N
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": updates / dt, "unit": "state-updates/s", "cores": cores, "kind": "oracle",
            "sample": f"{cb.size} of {Bn * D} channels (first {nd} channels of each of the "
                      f"{Bn} batch rows), all {L} steps, N={N}: {updates:.3e} updates in "
                      f"{dt:.1f} s on {cpu}"}


def variant_legs(ss, w, dev, args_f, keys, steps, with_cpu=False):
    """The strided-B/C, packed-sequence and complex variants, each timed on its
    own workload (see each leg's "workload")."""
    import torch
    out = {}
    B8, L8, D8, N8 = w.batch, w.seqlen, w.dim, w.dstate
    io = dev["u"].dtype
    ios = 2 if w.io_dtype != "f32" else 4
    fbytes = algorithmic_bytes(w)

    # B / C read in place from the x-projection output xdbl [B, L, dt_rank + 2N]
    # (dt_rank = 160 for d_model 2560), against gathering them first.
    R = 160
    xdbl = torch.randn(B8, L8, R + 2 * N8, generator=torch.Generator().manual_seed(7)).to(io).cuda()
    xdbl[..., R:R + N8] = dev["B"]
    xdbl[..., R + N8:] = dev["C"]
    y = torch.empty_like(dev["u"])
    sargs = list(args_f)
    sargs[keys.index("B")] = xdbl[..., R:R + N8]
    sargs[keys.index("C")] = xdbl[..., R + N8:]

    def s_step():
        ss.fwd(*sargs, y=y)

    def g_step():
        gargs = list(sargs)
        gargs[keys.index("B")] = sargs[keys.index("B")].contiguous()
        gargs[keys.index("C")] = sargs[keys.index("C")].contiguous()
        ss.fwd(*gargs, y=y)

    log("timing strided B/C")
    sms, _ = time_calls(s_step, steps, 2)
    gms, _ = time_calls(g_step, steps, 2)
    out["strided_bc"] = {
        "workload": "the 2.8B-shaped forward with B, C as column slices of xdbl "
                    f"[{B8}, {L8}, {R + 2 * N8}] (row stride {R + 2 * N8})",
        "us_per_call": sms * 1e3, "state_updates_per_s": w.updates / (sms * 1e-3),
        "us_per_call_gather_then_scan": gms * 1e3,
        "roofline": alu_roofline(w.updates / (sms * 1e-3), FLOPS_PER_UPDATE, (1, 4)),
    }
    log(f"strided {sms * 1e3:.1f} us, gather + scan {gms * 1e3:.1f} us")
    del xdbl, sargs

    # packed sequences: the same 16384 rows cut into 14 sequences of 256..2048 steps
    lens = [2048, 1024, 512, 2048, 1024, 512, 2048, 1024, 512, 2048, 1024, 512, 1024, 1024]
    assert sum(lens) == B8 * L8
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0)), dtype=torch.int32).cuda()
    pk = {k: (None if dev[k] is None else
              (dev[k].reshape(-1, dev[k].shape[-1]) if dev[k].dim() == 3 else dev[k]))
          for k in keys}
    yv = torch.empty_like(pk["u"])

    def v_step():
        ss.fwd_varlen(pk["u"], pk["delta"], pk["A"], pk["B"], pk["C"], cu, max(lens), pk["D"],
                      pk["z"], pk["delta_bias"], y=yv)

    log("timing packed sequences")
    vms, _ = time_calls(v_step, steps, 2)
    out["varlen"] = {
        "workload": f"the 2.8B-shaped forward's {B8 * L8} rows as {len(lens)} packed sequences "
                    f"of {min(lens)}..{max(lens)} steps (D=5120, N=16, bf16)",
        "us_per_call": vms * 1e3, "state_updates_per_s": w.updates / (vms * 1e-3),
        "hbm_gbs": fbytes / (vms * 1e-3) / 1e9,
        "roofline": alu_roofline(w.updates / (vms * 1e-3), FLOPS_PER_UPDATE, (1, 4)),
    }
    log(f"varlen {vms * 1e3:.1f} us")
    del pk, yv

    # complex A, B, C: forward and backward, B=2, L=2048, D=1024, N=16, f32
    Bc, Lc, Dc, Nc = 2, 2048, 1024, 16
    g = torch.Generator().manual_seed(11)
    f = lambda *sh: torch.randn(*sh, generator=g).cuda()
    cu_ = f(Bc, Lc, Dc)
    cdl = (f(Bc, Lc, Dc) * 0.5 - 1.0)
    cA = torch.stack([-torch.exp(torch.randn(Dc, Nc, generator=g)),
                      torch.randn(Dc, Nc, generator=g) * 2.0], -1).cuda()
    cB, cC = f(Bc, Lc, Nc, 2), f(Bc, Lc, Nc, 2)
    cD, cz, cbias, cdy = f(Dc), f(Bc, Lc, Dc), f(Dc) * 0.1 - 4.0, f(Bc, Lc, Dc)

    def cf_step():
        ss.fwd_complex(cu_, cdl, cA, cB, cC, cD, cz, cbias)

    def cb_step():
        ss.bwd_complex(cu_, cdl, cA, cB, cC, cD, cz, cbias, dy=cdy)

    log("timing complex")
    cfms, _ = time_calls(cf_step, steps, 2)
    cbms, _ = time_calls(cb_step, max(3, steps // 2), 1)
    upd = Bc * Lc * Dc * Nc
    cfb = (4 * Bc * Lc * Dc + 4 * Bc * Lc * Nc + Dc * Nc * 2 + 2 * Dc) * 4
    out["complex"] = {
        "workload": f"complex A/B/C, B={Bc}, L={Lc}, D={Dc}, N={Nc}, f32, D/z/delta_bias",
        "fwd_us_per_call": cfms * 1e3, "fwd_state_updates_per_s": upd / (cfms * 1e-3),
        "fwd_hbm_gbs": cfb / (cfms * 1e-3) / 1e9,
        "bwd_us_per_call": cbms * 1e3, "bwd_state_updates_per_s": upd / (cbms * 1e-3),
        "fwd_roofline": alu_roofline(upd / (cfms * 1e-3), FLOPS_PER_UPDATE_COMPLEX),
        "bwd_roofline": alu_roofline(upd / (cbms * 1e-3), FLOPS_PER_UPDATE_COMPLEX_BWD),
    }
    if with_cpu:
        import oracle
        log("timing the CPU oracle complex forward")
        cin = {"u": cu_.cpu(), "delta": cdl.cpu(), "A": cA.cpu(), "B": cB.cpu(), "C": cC.cpu(),
               "D": cD.cpu(), "z": cz.cpu(), "delta_bias": cbias.cpu()}

        def run_c(nd):
            oracle.fwd_complex(**{k: (v[..., :nd] if k in ("u", "delta", "z") else
                                      v[:nd] if k in ("A", "D", "delta_bias") else v)
                                  for k, v in cin.items()})

        out["complex"]["cpu_baseline"] = cpu_oracle_rate(
            run_c, Dc, Bc * Lc * Nc, 3.0, "numpy complex128 forward, all batch rows and steps")
    log(f"complex fwd {cfms * 1e3:.1f} us, bwd {cbms * 1e3:.1f} us")
    return out


CONFIG_NAMES = ("tiny", "m130m", "m2p8b", "long", "bwd")
# one GPU's share of an 8-way channel split of m2p8b and bwd (ss_inputs)
SHARD_NAMES = ("m2p8b_d8", "bwd_d8")


def rel_err(x, r) -> float:
    """max_i |x_i - r_i| / max(|r_i|, rms(r)) over one tensor (the parity metric)."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        return float(np.max(np.abs(x - r)))
    return float(np.max(np.abs(x - r) / np.maximum(np.abs(r), rms)))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def config_parity(ss, w, inp, args_f, dy, gpu_s: float) -> dict:
    """One workload against the float64 oracle: the max error per output, run-
    to-run bit-exactness (two calls compared bit for bit), and the oracle's
    time on the host cores (the whole workload, compute only)."""
    import torch
    import oracle
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")
    tol = 1e-5 if w.io_dtype == "f32" else 2e-2
    to64 = lambda t: t.detach().to("cpu", torch.float64).numpy()
    if w.backward:
        g1 = ss.bwd(*args_f, dy=dy)
        g2 = ss.bwd(*args_f, dy=dy)
        torch.cuda.synchronize()
        exact = all(torch.equal(g1[k], g2[k]) for k in g1 if g1[k] is not None)
        t0 = time.perf_counter()
        ref = oracle.bwd(**{k: inp[k] for k in keys}, dy=inp["dy"])
        osec = time.perf_counter() - t0
        errs = {k: rel_err(to64(g1[k]), ref[k]) for k in ref if ref[k] is not None}
    else:
        y1, l1 = ss.fwd(*args_f, return_last_state=True)
        y2, l2 = ss.fwd(*args_f, return_last_state=True)
        torch.cuda.synchronize()
        exact = torch.equal(y1, y2) and torch.equal(l1, l2)
        t0 = time.perf_counter()
        yr, lr = oracle.fwd(**{k: inp[k] for k in keys}, return_last_state=True)
        osec = time.perf_counter() - t0
        errs = {"y": rel_err(to64(y1), yr), "last_state": rel_err(to64(l1), lr)}
        del yr
    worst = max(errs.values())
    return {"max_rel_err": errs, "worst_rel_err": worst, "bound": tol, "within_bound": worst <= tol,
            "bit_exact_run_to_run": bool(exact),
            "oracle": {"seconds": osec, "cores": oracle.default_threads(), "cpu": cpu_model(),
                       "state_updates_per_s": w.updates / osec, "kind": "float64 C loop",
                       "gpu_speedup": osec / gpu_s}}


def configs_leg(ss, reps: int, names=CONFIG_NAMES, with_oracle: bool = True):
    """Every forward workload and the backward one, each timed per call warm
    (back to back) and cold (L2 and MALL evicted before every call): median,
    min and max, with updates/s and algorithmic GB/s at the cold median; with
    with_oracle, also each workload's parity record (config_parity)."""
    import torch
    from ss_inputs import WORKLOADS, make_inputs
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    out = {}
    for name in names:
        w = WORKLOADS[name]
        log(f"configs: {name}")
        inp = make_inputs(w)
        dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
        args_f = [dev[k] for k in keys]
        io = {"f32": 0, "f16": 1, "bf16": 2}[w.io_dtype]
        pa = {"f32": 0, "f16": 1, "bf16": 2}[w.param_dtype]
        desc = ss.SsDesc(w.batch, w.seqlen, w.dim, w.dstate, 1, io, pa, 0)
        if w.backward:
            ws = torch.empty(max(1, ss.workspace_size(desc, True)), dtype=torch.uint8,
                             device="cuda")

            def fn():
                ss.bwd(*args_f, dy=dev["dy"], workspace=ws)
            nbytes = algorithmic_bytes_bwd(w)
            launches = ss.plan(desc, True).n_launches
        else:
            ws = torch.empty(max(1, ss.workspace_size(desc)), dtype=torch.uint8, device="cuda")
            y = torch.empty_like(dev["u"])
            ls = (torch.empty(w.batch, w.dim, w.dstate, dtype=dev["A"].dtype, device="cuda")
                  if w.last_state else None)

            def fn():
                ss.fwd(*args_f, y=y, workspace=ws, last_state=ls)
            nbytes = algorithmic_bytes(w)
            launches = ss.plan(desc).n_launches
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        warm = time_each(fn, reps)
        cold = time_each(fn, reps, scratch)
        med = statistics.median(cold)
        out[name] = {
            "shape": f"B={w.batch}, L={w.seqlen}, D={w.dim}, N={w.dstate}, {w.io_dtype} io",
            "call": "ss_bwd" if w.backward else "ss_fwd", "launches": launches,
            "warm_us": {"median": statistics.median(warm) * 1e3, "min": min(warm) * 1e3,
                        "max": max(warm) * 1e3},
            "cold_us": {"median": med * 1e3, "min": min(cold) * 1e3, "max": max(cold) * 1e3},
            "state_updates_per_s_cold": w.updates / (med * 1e-3),
            "hbm_gbs_cold": nbytes / (med * 1e-3) / 1e9,
            "hbm_frac_cold": nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nbytes,
        }
        if with_oracle:
            log(f"configs: {name} against the oracle")
            out[name].update(config_parity(ss, w, inp, args_f, dev.get("dy"), med * 1e-3))
        del dev, args_f, ws, inp
        torch.cuda.empty_cache()
    del scratch
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed calls first (the clock settles within a few ms of load)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the strided-B/C, packed-sequence and complex legs")
    ap.add_argument("--variants-only", action="store_true",
                    help="time only those legs (for a kernel trace of them alone)")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the per-GPU shard shapes (D / 8 of m2p8b and bwd)")
    ap.add_argument("--no-state-sweep", action="store_true",
                    help="skip the forward / backward timings over N = 16 ... 256")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload warm / cold timings (and the shard shapes)")
    ap.add_argument("--configs-only", nargs="*", choices=CONFIG_NAMES + SHARD_NAMES, default=None,
                    metavar="NAME",
                    help="only the per-workload timings (of the named workloads, default all)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run a plain 512 MiB copy first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this benchmark runs on one GPU only (got --gpus {args.gpus}); the "
              "selective scan is timed at N=1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mamba_selective_scan_02_amd as ss
    from ss_inputs import WORKLOADS, make_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calib_copy:
        calibration_copy()
    if args.configs_only is not None:
        names = tuple(args.configs_only) or CONFIG_NAMES
        print(json.dumps({"configs": configs_leg(ss, args.steps, names,
                                                 not args.no_cpu_baseline)}), flush=True)
        return
    keys = ("u", "delta", "A", "B", "C", "D", "z", "delta_bias")
    w = WORKLOADS["m2p8b"]
    log(f"generating {w.name} inputs")
    inp = make_inputs(w)
    dev = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    args_f = [dev[k] for k in keys]
    y = torch.empty_like(dev["u"])
    desc = ss.SsDesc(w.batch, w.seqlen, w.dim, w.dstate, 1, 2, 0, 0)
    plan = ss.plan(desc)
    ws = torch.empty(max(1, ss.workspace_size(desc)), dtype=torch.uint8, device="cuda")

    def step():
        ss.fwd(*args_f, y=y, workspace=ws)

    if args.variants_only:
        print(json.dumps(variant_legs(ss, w, dev, args_f, keys, args.steps)), flush=True)
        return
    # The headline step: warmup, then K calls each timed by its own HIP events
    # on the launch stream, with L2 and the 256 MB MALL evicted before every
    # call (time_each), so each call reads its inputs from HBM; the value is
    # taken at the median.  The same K calls back to back are reported beside
    # it.
    log(f"timing forward: warmup {args.warmup}, steps {args.steps}")
    for _ in range(args.warmup):
        step()
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    cold = time_each(step, args.steps, scratch)
    wall = time.perf_counter() - t_wall
    del scratch
    warm_ms, _ = time_calls(step, args.steps, 1)
    ms = statistics.median(cold)
    updates = w.updates
    value = updates / (ms * 1e-3)
    abytes = algorithmic_bytes(w)
    gbs = abytes / (ms * 1e-3) / 1e9
    log(f"forward {ms * 1e3:.1f} us/step (median, cold), {value:.3e} updates/s, {gbs:.0f} GB/s; "
        f"back to back {warm_ms * 1e3:.1f} us")

    result = {
        "metric": "selective_scan fwd state-updates/s and HBM GB/s (% of peak), 1 MI355X",
        "value": value,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "Mamba-2.8B-shaped selective_scan forward: B=8, L=2048, D=5120, "
                               "N=16, bf16 u/delta/B/C/z/y, f32 A/D/delta_bias, softplus on",
                   "batch": w.batch, "seq_len": w.seqlen, "dim": w.dim, "dstate": w.dstate,
                   "io_dtype": w.io_dtype, "param_dtype": w.param_dtype,
                   "n_chunks": plan.n_chunks, "kernels_per_step": plan.n_launches},
        "timing": {"protocol": "median of K calls, L2 and MALL evicted (1 GiB read) before each",
                   "us_min": min(cold) * 1e3, "us_max": max(cold) * 1e3,
                   "us_per_call_back_to_back": warm_ms * 1e3,
                   "state_updates_per_s_back_to_back": updates / (warm_ms * 1e-3)},
        "hbm_gbs": gbs,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "algorithmic_bytes": abytes,
        # binding roofline: the update's instruction mix (1 transcendental +
        # 4 FP32 ops) at the ALU peak; the HBM and FP32-vector fractions beside it
        "roofline": dict(alu_roofline(value, FLOPS_PER_UPDATE, (1, 4)),
                         kernel="fwd_wide (single pass, 8 lanes per channel, LDS-staged streams)",
                         traffic=stored_traffic("fwd_wide_m2p8b"),
                         hbm_achieved_gbs=gbs, hbm_peak_gbs=HBM_PEAK_GBS,
                         hbm_frac=gbs / HBM_PEAK_GBS,
                         floors_us={"hbm": abytes / (HBM_PEAK_GBS * 1e9) * 1e6,
                                    "fp32_vector": updates * FLOPS_PER_UPDATE
                                    / (FP32_VECTOR_PEAK_TFLOPS * 1e12) * 1e6,
                                    "alu_mix": updates / mix_peak_updates(1, 4) * 1e6,
                                    "measured_update_mix": updates / MEASURED_UPDATE_MIX * 1e6},
                         measured_mix_frac=value / MEASURED_UPDATE_MIX),
        "wall_s": wall,
    }
    del y, ws

    if not args.no_bwd:
        wb = WORKLOADS["bwd"]
        log("generating bwd inputs")
        ib = make_inputs(wb)
        db = {k: (None if v is None else v.cuda()) for k, v in ib.items()}
        descb = ss.SsDesc(wb.batch, wb.seqlen, wb.dim, wb.dstate, 1, 0, 0, 0)
        wsb = torch.empty(max(1, ss.workspace_size(descb, True)), dtype=torch.uint8,
                          device="cuda")
        argsb = [db[k] for k in keys]

        def bstep():
            ss.bwd(*argsb, dy=db["dy"], workspace=wsb)

        bsteps = max(3, args.steps // 2)
        log(f"timing backward: steps {bsteps}")
        bms, _ = time_calls(bstep, bsteps, max(1, args.warmup))
        bb = algorithmic_bytes_bwd(wb)
        result["backward"] = {
            "workload": "B=2, L=2048, D=2048, N=16, f32, D/z/delta_bias, dy",
            "ms_per_call": bms, "state_updates_per_s": wb.updates / (bms * 1e-3),
            "hbm_gbs": bb / (bms * 1e-3) / 1e9, "hbm_frac": bb / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": bb,
            "n_kernels": ss.plan(descb, True).n_launches,
            "traffic": stored_traffic("ss_bwd_bwd"),
            "roofline": alu_roofline(wb.updates / (bms * 1e-3), FLOPS_PER_UPDATE_BWD, (3, 20)),
        }
        if not args.no_cpu_baseline:
            import oracle
            log("timing the CPU oracle backward")

            def run_b(nd):
                sub = {k: (None if ib[k] is None else
                           (ib[k][..., :nd] if k in ("u", "delta", "z", "dy") else
                            ib[k][:nd] if k in ("A", "D", "delta_bias") else ib[k]))
                       for k in keys + ("dy",)}
                oracle.bwd(**sub)

            result["backward"]["cpu_baseline"] = cpu_oracle_rate(
                run_b, wb.dim, wb.batch * wb.seqlen * wb.dstate, 5.0,
                "float64 C backward, all batch rows and steps")
        log(f"backward {bms * 1e3:.1f} us/call")
        del wsb, db

    if not args.no_decode:
        # One recurrence step on a carried state, updated in place (ss_fwd_h0
        # with L = 1 and last_state == h0), for the 2.8B-shaped layer: the
        # first step of the forward inputs, a seeded N(0, 1) f32 state.
        B8, D8, N8 = w.batch, w.dim, w.dstate
        step_args = [None if t is None else (t[:, :1].contiguous() if t.dim() == 3 else t)
                     for t in args_f]
        gen = torch.Generator().manual_seed(2024)
        state = torch.randn(B8, D8, N8, generator=gen).cuda()
        ys = torch.empty((B8, 1, D8), dtype=dev["u"].dtype, device="cuda")

        def dstep():
            ss.fwd(*step_args, y=ys, h0=state, last_state=state)

        dsteps = 200
        log(f"timing decode step: {dsteps} steps")
        dms, _ = time_calls(dstep, dsteps, 20)
        # The same steps replayed from a HIP graph of 20 steps: what a serving
        # loop pays per step once the host-side call overhead is gone.
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            dstep()
            with torch.cuda.graph(graph):
                for _ in range(20):
                    dstep()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        gms, _ = time_calls(graph.replay, 10, 2)
        gms /= 20
        io2 = 2 if w.io_dtype != "f32" else 4
        dbytes = (2 * B8 * D8 * N8 * 4 + 4 * B8 * D8 * io2 + 2 * B8 * N8 * io2 + D8 * N8 * 4
                  + 2 * D8 * 4)
        result["decode"] = {
            "workload": "one step of the 2.8B-shaped layer on a carried state: B=8, D=5120, "
                        "N=16, bf16 u/delta/z/y/B/C, f32 A/D/delta_bias/state, in place",
            "us_per_step": dms * 1e3, "tokens_per_s": B8 / (dms * 1e-3),
            "us_per_step_graph": gms * 1e3, "tokens_per_s_graph": B8 / (gms * 1e-3),
            "state_updates_per_s": B8 * D8 * N8 / (dms * 1e-3),
            "algorithmic_bytes": dbytes, "hbm_gbs": dbytes / (dms * 1e-3) / 1e9,
            "hbm_frac": dbytes / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            # one step moves 5.9 MB in a few microseconds: bound by HBM and
            # launch latency, priced here against HBM at the graph-replay rate
            "roofline": {"bound": "hbm", "achieved": dbytes / (gms * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        }
        log(f"decode {dms * 1e3:.2f} us/step, {gms * 1e3:.2f} us/step from a graph")
        del state

    if not args.no_variants:
        result.update(variant_legs(ss, w, dev, args_f, keys, max(5, args.steps // 2),
                                   with_cpu=not args.no_cpu_baseline))

    if not args.no_configs:
        result["configs"] = configs_leg(ss, args.steps, with_oracle=not args.no_cpu_baseline)
    if not args.no_configs and not args.no_shard:
        # What one GPU of an 8-GPU node runs when the channels are split 8
        # ways: the forward needs no communication there, so 8 x its rate is
        # the node's forward rate on the full m2p8b problem; the backward adds
        # one fixed-order sum of dB / dC over the GPUs (not measured here).
        sh = configs_leg(ss, args.steps, SHARD_NAMES, with_oracle=not args.no_cpu_baseline)
        for name, full in (("m2p8b_d8", "m2p8b"), ("bwd_d8", "bwd")):
            sh[name]["share_of"] = f"{full} split 8 ways over D"
            sh[name]["node_state_updates_per_s_8_gpus"] = 8 * sh[name]["state_updates_per_s_cold"]
        result["shard"] = sh

    if not args.no_state_sweep:
        result["state_sweep"] = state_sweep_leg(ss, max(5, args.steps // 2))

    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
