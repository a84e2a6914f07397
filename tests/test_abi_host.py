"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/ss.h declares, and
reject invalid calls with the right status before touching the device:
the validation rules of the baracuda-kernels page
src/attention/selective_scan.rs (SelectiveScanPlan::select / can_implement,
the backward plan's run: non-negative extents, dstate <= 256, f32/f16/bf16,
workspace size, optional-input / gradient presence pairs).  No call here
reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

import mamba_selective_scan_02_amd as ss

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss.h")

# A fake, suitably aligned "device" address: validation only inspects it.
P = ctypes.c_void_p(0x7F0000000000)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ss_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ss.load_library()
    names = _declared_functions()
    assert set(names) == {"ss_workspace_size", "ss_fwd", "ss_bwd", "ss_fwd_h0", "ss_bwd_h0",
                          "ss_bwd_noalloc", "ss_fwd_varlen", "ss_bwd_varlen", "ss_fwd_strided",
                          "ss_bwd_strided", "ss_workspace_size_complex", "ss_fwd_complex",
                          "ss_bwd_complex", "ss_plan_query",
                          "ss_status_string",
                          "ss_last_error"}
    for n in names:
        assert hasattr(lib, n), n


def _desc(B=2, L=64, D=96, N=16, sp=1, io=ss.SS_F32, pa=ss.SS_F32, chunk=0):
    return ss.SsDesc(B, L, D, N, sp, io, pa, chunk)


def _fwd(desc, **over):
    args = dict(u=P, delta=P, A=P, B=P, C=P, Dskip=None, z=None, delta_bias=None, y=P,
                last_state=None, workspace=None, workspace_bytes=0)
    args.update(over)
    return ss.ss_fwd(desc, args["u"], args["delta"], args["A"], args["B"], args["C"],
                     args["Dskip"], args["z"], args["delta_bias"], args["y"],
                     args["last_state"], args["workspace"], args["workspace_bytes"], None)


def _bwd(desc, **over):
    args = dict(u=P, delta=P, A=P, B=P, C=P, Dskip=None, z=None, delta_bias=None, dy=P,
                du=P, ddelta=P, dA=P, dB=P, dC=P, dD=None, dz=None, ddelta_bias=None,
                workspace=P, workspace_bytes=1 << 40)
    args.update(over)
    return ss.ss_bwd(desc, *[args[k] for k in ("u", "delta", "A", "B", "C", "Dskip", "z",
                                               "delta_bias", "dy", "du", "ddelta", "dA", "dB",
                                               "dC", "dD", "dz", "ddelta_bias", "workspace")],
                     args["workspace_bytes"], None)


def _fwd_h0(desc, h0, last_state):
    return ss.ss_fwd_h0(desc, P, P, P, P, P, None, None, None, h0, P, last_state, None, 0, None)


def _bwd_h0(desc, h0, dh0):
    return ss.ss_bwd_h0(desc, P, P, P, P, P, None, None, None, h0, P, P, P, P, P, P, None, None,
                        None, dh0, P, 1 << 40, None)


def test_h0_rules():
    d = _desc()                                   # B=2, D=96, N=16: a state is 12 KiB in f32
    q = ctypes.c_void_p(0x7F0000100000)
    # h0 and dh0 come together
    assert _bwd_h0(d, P, None) == ss.SS_ERR_INVALID_PROBLEM
    assert "h0 and dh0" in ss.ss_last_error()
    assert _bwd_h0(d, None, P) == ss.SS_ERR_INVALID_PROBLEM
    # alignment to the parameter element size
    odd = ctypes.c_void_p(0x7F0000000002)
    assert _fwd_h0(d, odd, None) == ss.SS_ERR_INVALID_PROBLEM
    assert "h0" in ss.ss_last_error()
    # last_state may be h0 itself, never a partial overlap
    assert _fwd_h0(d, P, ctypes.c_void_p(0x7F0000000000 + 256)) == ss.SS_ERR_INVALID_PROBLEM
    assert "overlap" in ss.ss_last_error()
    assert _bwd_h0(d, P, ctypes.c_void_p(0x7F0000000000 + 4)) == ss.SS_ERR_INVALID_PROBLEM
    assert "overlap" in ss.ss_last_error()
    # disjoint buffers pass validation up to the workspace check
    ws = ss.ss_workspace_size(d, 0)
    if ws > 0:
        assert _fwd_h0(d, P, q) == ss.SS_ERR_WORKSPACE_TOO_SMALL


def test_varlen_rules():
    d = _desc()
    call = lambda cu, total: ss.ss_fwd_varlen(d, cu, total, P, P, P, P, P, None, None, None,
                                              None, P, None, None, 0, None)
    assert call(None, 10) == ss.SS_ERR_INVALID_PROBLEM
    assert "cu_seqlens" in ss.ss_last_error()
    assert call(ctypes.c_void_p(0x7F0000000002), 10) == ss.SS_ERR_INVALID_PROBLEM
    assert "aligned" in ss.ss_last_error()
    assert call(P, -1) == ss.SS_ERR_INVALID_PROBLEM
    assert "total_len" in ss.ss_last_error()
    # more rows than batch * seqlen
    assert call(P, 2 * 64 + 1) == ss.SS_ERR_INVALID_PROBLEM
    assert "batch * seqlen" in ss.ss_last_error()
    bcall = lambda cu, total: ss.ss_bwd_varlen(d, cu, total, P, P, P, P, P, None, None, None,
                                               None, P, P, P, P, P, P, None, None, None, None,
                                               P, 1 << 40, None)
    assert bcall(None, 10) == ss.SS_ERR_INVALID_PROBLEM
    assert "cu_seqlens" in ss.ss_last_error()
    assert bcall(ctypes.c_void_p(0x7F0000000002), 10) == ss.SS_ERR_INVALID_PROBLEM
    assert bcall(P, -1) == ss.SS_ERR_INVALID_PROBLEM
    assert bcall(P, 2 * 64 + 1) == ss.SS_ERR_INVALID_PROBLEM
    assert "batch * seqlen" in ss.ss_last_error()
    # h0 / dh0 still come together
    assert ss.ss_bwd_varlen(d, P, 10, P, P, P, P, P, None, None, None, P, P, P, P, P, P, P,
                            None, None, None, None, P, 1 << 40, None) == ss.SS_ERR_INVALID_PROBLEM


def test_strided_rules():
    # every call below stops in validation (no launch): the workspace is
    # always too small for shapes that pass the stride checks
    q = ctypes.c_void_p(0x7F0000100000)

    def fcall(d, ldb, ldc, cu=None, total=0):
        return ss.ss_fwd_strided(d, cu, total, ldb, ldc, P, P, P, P, P, None, None, None, None,
                                 P, None, q, 0, None)

    def bcall(d, ldb, ldc):
        return ss.ss_bwd_strided(d, None, 0, ldb, ldc, P, P, P, P, P, None, None, None, None, P,
                                 P, P, P, P, P, None, None, None, None, P, 0, None)

    d = _desc(B=1, L=4096, D=64, N=16)             # chunked: needs a forward workspace
    assert ss.ss_workspace_size(d, 0) > 0
    # strides below N
    assert fcall(d, 15, 16) == ss.SS_ERR_INVALID_PROBLEM
    assert "stride" in ss.ss_last_error()
    assert fcall(d, 16, 8) == ss.SS_ERR_INVALID_PROBLEM
    assert bcall(d, 16, 3) == ss.SS_ERR_INVALID_PROBLEM
    # strides that fit pass validation up to the workspace check
    assert fcall(d, 0, 0) == ss.SS_ERR_WORKSPACE_TOO_SMALL
    assert fcall(d, 192, 200) == ss.SS_ERR_WORKSPACE_TOO_SMALL
    assert bcall(d, 192, 192) == ss.SS_ERR_WORKSPACE_TOO_SMALL
    # a single 4096-step chunk of a 2^20-element stride exceeds the tile
    # kernels' 32-bit offsets; shorter forced chunks lift that
    big = _desc(B=8, L=4096, D=5120, N=16, io=ss.SS_BF16)
    assert ss.plan(big).n_chunks == 1
    assert fcall(big, 1 << 20, 16) == ss.SS_ERR_UNSUPPORTED
    assert "chunk_len" in ss.ss_last_error()
    short = _desc(B=8, L=4096, D=5120, N=16, io=ss.SS_BF16, chunk=256)
    assert fcall(short, 1 << 20, 16) == ss.SS_ERR_WORKSPACE_TOO_SMALL
    # the varlen rules apply when cu_seqlens is given
    assert fcall(d, 192, 192, P, -1) == ss.SS_ERR_INVALID_PROBLEM
    assert "total_len" in ss.ss_last_error()
    assert fcall(d, 192, 192, P, 4097) == ss.SS_ERR_INVALID_PROBLEM


def test_complex_rules():
    d = _desc(B=1, L=4096, D=64, N=16)
    fcall = lambda ws_bytes, **kw: ss.ss_fwd_complex(
        d, P, P, P, P, P, None, None, None, kw.get("h0"), P, kw.get("ls"), P, ws_bytes, None)
    bcall = lambda **kw: ss.ss_bwd_complex(
        d, P, P, P, P, P, kw.get("Dskip"), None, None, kw.get("h0"), P, P, P, P, P, P,
        kw.get("dD"), None, None, kw.get("dh0"), P, 0, None)
    # the complex workspace holds (re, im) states: larger than the real one
    wf, wb = ss.ss_workspace_size_complex(d, 0), ss.ss_workspace_size_complex(d, 1)
    assert wf > ss.ss_workspace_size(d, 0) > 0 and wb > 0
    assert fcall(wf - 1) == ss.SS_ERR_WORKSPACE_TOO_SMALL
    assert str(wf) in ss.ss_last_error()
    assert bcall() == ss.SS_ERR_WORKSPACE_TOO_SMALL
    assert bcall(h0=P) == ss.SS_ERR_INVALID_PROBLEM
    assert "h0 and dh0" in ss.ss_last_error()
    assert bcall(Dskip=P) == ss.SS_ERR_INVALID_PROBLEM
    # h0 / last_state: same buffer or disjoint (a state is 2 * 64 * 16 floats)
    assert fcall(wf, h0=P, ls=ctypes.c_void_p(0x7F0000000000 + 8)) == ss.SS_ERR_INVALID_PROBLEM
    assert "overlap" in ss.ss_last_error()
    assert ss.ss_workspace_size_complex(_desc(N=257), 0) == 0
    assert ss.ss_fwd_complex(_desc(N=257), P, P, P, P, P, None, None, None, None, P, None, None,
                             0, None) == ss.SS_ERR_UNSUPPORTED


def test_status_strings():
    assert ss.ss_status_string(ss.SS_OK) == "success"
    assert "invalid" in ss.ss_status_string(ss.SS_ERR_INVALID_PROBLEM)
    assert "unsupported" in ss.ss_status_string(ss.SS_ERR_UNSUPPORTED)
    assert "workspace" in ss.ss_status_string(ss.SS_ERR_WORKSPACE_TOO_SMALL)
    assert ss.ss_status_string(99) == "unknown status"


@pytest.mark.parametrize("field", ["batch", "seqlen", "dim", "dstate"])
def test_negative_extent_is_invalid(field):
    d = _desc()
    setattr(d, field, -1)
    assert _fwd(d) == ss.SS_ERR_INVALID_PROBLEM
    assert "non-negative" in ss.ss_last_error()
    assert _bwd(d) == ss.SS_ERR_INVALID_PROBLEM
    assert ss.ss_workspace_size(d, 0) == 0


def test_dstate_limit():
    assert _fwd(_desc(N=257)) == ss.SS_ERR_UNSUPPORTED
    assert "256" in ss.ss_last_error()
    assert _bwd(_desc(N=257)) == ss.SS_ERR_UNSUPPORTED


def test_dtypes():
    assert _fwd(_desc(io=3)) == ss.SS_ERR_UNSUPPORTED
    assert _fwd(_desc(io=ss.SS_BF16, pa=ss.SS_F16)) == ss.SS_ERR_UNSUPPORTED
    assert _fwd(_desc(io=ss.SS_F16, pa=ss.SS_BF16)) == ss.SS_ERR_UNSUPPORTED
    assert _fwd(_desc(sp=2)) == ss.SS_ERR_INVALID_PROBLEM
    assert _fwd(_desc(chunk=-4)) == ss.SS_ERR_INVALID_PROBLEM
    assert _fwd(None) == ss.SS_ERR_INVALID_PROBLEM


@pytest.mark.parametrize("name", ["u", "delta", "A", "B", "C", "y"])
def test_null_required_pointer(name):
    assert _fwd(_desc(chunk=1 << 20), **{name: None}) == ss.SS_ERR_INVALID_PROBLEM
    assert "NULL" in ss.ss_last_error()


def test_misaligned_pointer():
    bad = ctypes.c_void_p(0x7F0000000002)
    assert _fwd(_desc(chunk=1 << 20), u=bad) == ss.SS_ERR_INVALID_PROBLEM
    assert "aligned" in ss.ss_last_error()
    # 2-byte alignment is enough for 16-bit io
    d = _desc(io=ss.SS_BF16, chunk=1 << 20)
    assert _fwd(d, last_state=ctypes.c_void_p(0x7F0000000001)) == ss.SS_ERR_INVALID_PROBLEM


def test_workspace_too_small():
    # a shape that needs the chunked (two-level) forward
    d = _desc(B=1, L=4096, D=64, N=16)
    need = ss.ss_workspace_size(d, 0)
    assert need > 0
    assert _fwd(d, workspace=P, workspace_bytes=need - 1) == ss.SS_ERR_WORKSPACE_TOO_SMALL
    assert str(need) in ss.ss_last_error()
    assert _fwd(d, workspace=None, workspace_bytes=need) == ss.SS_ERR_INVALID_PROBLEM
    assert _fwd(d, workspace=ctypes.c_void_p(0x7F0000000010),
                workspace_bytes=need) == ss.SS_ERR_INVALID_PROBLEM
    db = _desc(B=1, L=4096, D=64, N=16)
    needb = ss.ss_workspace_size(db, 1)
    assert _bwd(db, workspace_bytes=needb - 1) == ss.SS_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("pair", [("Dskip", "dD"), ("z", "dz"), ("delta_bias", "ddelta_bias")])
def test_backward_presence_pairs(pair):
    a, b = pair
    assert _bwd(_desc(), **{a: P}) == ss.SS_ERR_INVALID_PROBLEM
    assert "both given or both omitted" in ss.ss_last_error()
    assert _bwd(_desc(), **{b: P}) == ss.SS_ERR_INVALID_PROBLEM


def test_empty_problem_is_a_noop():
    for field in ("batch", "seqlen", "dim"):
        d = _desc()
        setattr(d, field, 0)
        # no pointers at all: nothing is read or written, nothing launched
        assert _fwd(d, u=None, delta=None, A=None, B=None, C=None, y=None) == ss.SS_OK
        assert ss.ss_workspace_size(d, 0) == 0
        assert ss.plan(d, False).n_launches == 0


def test_plan_is_a_function_of_shape():
    # large B * D: single pass
    p = ss.plan(_desc(B=8, L=2048, D=5120, N=16, io=ss.SS_BF16))
    assert (p.n_chunks, p.n_launches, p.states_per_lane, p.lanes_per_channel) == (1, 1, 2, 8)
    assert ss.ss_workspace_size(_desc(B=8, L=2048, D=5120, N=16, io=ss.SS_BF16), 0) == 0
    # small B * D, long L: chunked two-level scan
    p = ss.plan(_desc(B=1, L=262144, D=512, N=16))
    assert p.n_chunks > 1 and p.n_launches == 3
    assert p.chunk_len * p.n_chunks >= 262144 > p.chunk_len * (p.n_chunks - 1)
    # forced chunk length
    p = ss.plan(_desc(B=1, L=100, D=32, N=16, chunk=7))
    assert (p.chunk_len, p.n_chunks) == (7, 15)
    # N buckets
    for n, (ns, g) in {0: (1, 8), 1: (1, 8), 5: (1, 8), 9: (2, 8), 16: (2, 8), 17: (4, 8),
                       32: (4, 8), 33: (8, 8), 64: (8, 8), 65: (16, 8), 128: (16, 8),
                       200: (16, 16), 256: (16, 16)}.items():
        p = ss.plan(_desc(N=n))
        assert (p.states_per_lane, p.lanes_per_channel) == (ns, g), n
    # N > 64 short of its lanes' states: B / C copied into padded rows first
    # (one more launch, two [B * L, NS * G] buffers in the workspace)
    d100, d128 = _desc(B=2, L=300, D=64, N=100), _desc(B=2, L=300, D=64, N=128)
    assert ss.plan(d100).n_launches == ss.plan(d128).n_launches + 1
    assert ss.ss_workspace_size(d100, 0) >= 2 * (2 * 300 * 128 * 4)
    # backward: N <= 16 uses the tile kernels with chunks of 64 steps, N <= 32
    # the tile kernels with 4 states per lane and chunks of 32 steps, larger N
    # the general kernels with chunks of 8 steps
    p = ss.plan(_desc(B=2, L=2048, D=2048, N=16), True)
    assert (p.chunk_len, p.n_chunks, p.n_launches, p.states_per_lane,
            p.lanes_per_channel) == (64, 32, 4, 2, 8)
    for n in (17, 32):
        p = ss.plan(_desc(B=2, L=2048, D=2048, N=n), True)
        assert (p.chunk_len, p.n_chunks, p.n_launches, p.states_per_lane,
                p.lanes_per_channel) == (32, 64, 4, 4, 8), n
    p = ss.plan(_desc(B=2, L=2048, D=2048, N=33), True)
    assert (p.chunk_len, p.n_chunks, p.n_launches) == (8, 256, 4)


def test_workspace_size_formula():
    B, L, D, N = 1, 4096, 64, 16
    d = _desc(B=B, L=L, D=D, N=N)
    p = ss.plan(d)
    K = p.n_chunks
    al = lambda x: (x + 255) // 256 * 256
    assert ss.ss_workspace_size(d, 0) == al(4 * B * K * D) + al(4 * B * K * N * D)


def test_noalloc_rejects_problems_beyond_its_scratch():
    """ss_bwd_noalloc refuses a problem whose workspace exceeds its static
    scratch (64 MiB) before touching the device, and names both sizes."""
    big = _desc(B=8, L=2048, D=5120, N=16)
    need = ss.ss_workspace_size(big, 1)
    assert need > 64 << 20
    st = ss.ss_bwd_noalloc(big, P, P, P, P, P, None, None, None, None, P, P, P, P, P, P, None,
                           None, None, None, None)
    assert st == ss.SS_ERR_UNSUPPORTED
    msg = ss.ss_last_error()
    assert "ss_bwd_noalloc" in msg and str(need) in msg and str(64 << 20) in msg
    # invalid descriptors are reported as by the other entry points
    st = ss.ss_bwd_noalloc(_desc(B=-1), P, P, P, P, P, None, None, None, None, P, P, P, P, P,
                           P, None, None, None, None, None)
    assert st == ss.SS_ERR_INVALID_PROBLEM
    # the backward workload's workspace fits the scratch
    assert ss.ss_workspace_size(_desc(B=2, L=2048, D=2048, N=16), 1) <= 64 << 20
