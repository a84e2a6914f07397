"""Mamba-1 selective scan on AMD Instinct MI355X (gfx950).

A thin binding over the C library ``libss.so`` (declared in ``include/ss.h``).
Every step of the computation runs in the library's HIP kernels; this module
only validates Python arguments, allocates outputs and workspace with torch
on the tensors' device and passes raw pointers plus the current HIP stream.
If the library is missing, every call raises: there is no fallback.

Raw C entry points with the header's names: ``ss_workspace_size``,
``ss_fwd``, ``ss_bwd``, ``ss_fwd_h0``, ``ss_bwd_h0``, ``ss_bwd_noalloc``, ``ss_fwd_varlen``,
``ss_bwd_varlen``, ``ss_fwd_strided``, ``ss_bwd_strided``,
``ss_workspace_size_complex``, ``ss_fwd_complex``, ``ss_bwd_complex``,
``ss_plan_query``, ``ss_status_string``, ``ss_last_error``.  Tensor-level
helpers: ``fwd``, ``bwd`` (both with an optional initial state ``h0``),
``fwd_varlen`` / ``bwd_varlen`` (packed variable-length sequences),
``fwd_complex`` / ``bwd_complex`` (complex A, B, C and state),
``decode_step`` and the autograd function ``selective_scan``.  B and C (and
the dB / dC outputs) may be row-strided views, e.g. column slices of the
x-projection output; those calls go to the strided entry points.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

__all__ = ["SsDesc", "SsPlan", "fwd", "bwd", "fwd_varlen", "bwd_varlen", "decode_step",
           "selective_scan", "plan", "workspace_size", "ss_workspace_size", "ss_fwd", "ss_bwd",
           "ss_fwd_h0", "ss_bwd_h0", "ss_bwd_noalloc", "ss_fwd_varlen", "ss_bwd_varlen", "ss_fwd_strided",
           "ss_bwd_strided", "ss_workspace_size_complex", "ss_fwd_complex", "ss_bwd_complex",
           "fwd_complex", "bwd_complex",
           "ss_plan_query", "ss_status_string",
           "ss_last_error", "library_path", "load_library",
           "SS_OK", "SS_ERR_INVALID_PROBLEM", "SS_ERR_UNSUPPORTED",
           "SS_ERR_WORKSPACE_TOO_SMALL", "SS_ERR_HIP"]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libss.so")

SS_F32, SS_F16, SS_BF16 = 0, 1, 2
SS_OK, SS_ERR_INVALID_PROBLEM, SS_ERR_UNSUPPORTED, SS_ERR_WORKSPACE_TOO_SMALL, SS_ERR_HIP = range(5)

_DTYPE_ID = {torch.float32: SS_F32, torch.float16: SS_F16, torch.bfloat16: SS_BF16}


class SsDesc(ctypes.Structure):
    """Mirror of ``ss_desc``."""
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("dstate", ctypes.c_int32),
                ("delta_softplus", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("param_dtype", ctypes.c_int32), ("chunk_len", ctypes.c_int32)]


class SsPlan(ctypes.Structure):
    """Mirror of ``ss_plan``."""
    _fields_ = [("chunk_len", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
                ("states_per_lane", ctypes.c_int32), ("lanes_per_channel", ctypes.c_int32),
                ("n_launches", ctypes.c_int32)]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libss.so (once).  Raises if it has not been built.  The
    SS_LIBRARY environment variable names another build of the same library
    (the sanitizer build of the host code, tests/test_sanitizers.py)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or os.environ.get("SS_LIBRARY") or library_path
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with "
                           "`python -m mamba_selective_scan_02_amd.build`")
    lib = ctypes.CDLL(p)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(SsDesc)
    lib.ss_workspace_size.argtypes = [dp, ctypes.c_int32]
    lib.ss_workspace_size.restype = sz
    lib.ss_fwd.argtypes = [dp] + [vp] * 11 + [sz, vp]
    lib.ss_fwd.restype = ctypes.c_int
    lib.ss_bwd.argtypes = [dp] + [vp] * 18 + [sz, vp]
    lib.ss_bwd.restype = ctypes.c_int
    lib.ss_fwd_h0.argtypes = [dp] + [vp] * 12 + [sz, vp]
    lib.ss_fwd_h0.restype = ctypes.c_int
    lib.ss_bwd_h0.argtypes = [dp] + [vp] * 20 + [sz, vp]
    lib.ss_bwd_h0.restype = ctypes.c_int
    lib.ss_bwd_noalloc.argtypes = [dp] + [vp] * 20
    lib.ss_bwd_noalloc.restype = ctypes.c_int
    lib.ss_fwd_varlen.argtypes = [dp, vp, ctypes.c_int64] + [vp] * 12 + [sz, vp]
    lib.ss_fwd_varlen.restype = ctypes.c_int
    lib.ss_bwd_varlen.argtypes = [dp, vp, ctypes.c_int64] + [vp] * 20 + [sz, vp]
    lib.ss_bwd_varlen.restype = ctypes.c_int
    i64 = ctypes.c_int64
    lib.ss_fwd_strided.argtypes = [dp, vp, i64, i64, i64] + [vp] * 12 + [sz, vp]
    lib.ss_fwd_strided.restype = ctypes.c_int
    lib.ss_bwd_strided.argtypes = [dp, vp, i64, i64, i64] + [vp] * 20 + [sz, vp]
    lib.ss_bwd_strided.restype = ctypes.c_int
    lib.ss_workspace_size_complex.argtypes = [dp, ctypes.c_int32]
    lib.ss_workspace_size_complex.restype = sz
    lib.ss_fwd_complex.argtypes = [dp] + [vp] * 12 + [sz, vp]
    lib.ss_fwd_complex.restype = ctypes.c_int
    lib.ss_bwd_complex.argtypes = [dp] + [vp] * 20 + [sz, vp]
    lib.ss_bwd_complex.restype = ctypes.c_int
    lib.ss_plan_query.argtypes = [dp, ctypes.c_int32, ctypes.POINTER(SsPlan)]
    lib.ss_plan_query.restype = ctypes.c_int
    lib.ss_status_string.argtypes = [ctypes.c_int]
    lib.ss_status_string.restype = ctypes.c_char_p
    lib.ss_last_error.argtypes = []
    lib.ss_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ----------------------------------------------------------- raw C entry points

def _ref(desc):
    return None if desc is None else ctypes.byref(desc)


def ss_workspace_size(desc: SsDesc, backward: int) -> int:
    return load_library().ss_workspace_size(_ref(desc), int(backward))


def ss_fwd(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, y, last_state,
           workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_fwd(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias,
                                 y, last_state, workspace, workspace_bytes, stream)


def ss_bwd(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, dy, du, ddelta, dA, dB, dC,
           dD, dz, ddelta_bias, workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_bwd(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias,
                                 dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, workspace,
                                 workspace_bytes, stream)


def ss_fwd_h0(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, h0, y, last_state,
              workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_fwd_h0(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias, h0,
                                    y, last_state, workspace, workspace_bytes, stream)


def ss_bwd_h0(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, h0, dy, du, ddelta, dA,
              dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_bwd_h0(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias, h0,
                                    dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                                    workspace, workspace_bytes, stream)


def ss_bwd_noalloc(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, h0, dy, du, ddelta,
                   dA, dB, dC, dD, dz, ddelta_bias, dh0, stream) -> int:
    return load_library().ss_bwd_noalloc(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias,
                                         h0, dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                                         dh0, stream)


def ss_fwd_varlen(desc: SsDesc, cu_seqlens, total_len: int, u, delta, A, B, C, Dskip, z,
                  delta_bias, h0, y, last_state, workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_fwd_varlen(_ref(desc), cu_seqlens, int(total_len), u, delta, A, B,
                                        C, Dskip, z, delta_bias, h0, y, last_state, workspace,
                                        workspace_bytes, stream)


def ss_bwd_varlen(desc: SsDesc, cu_seqlens, total_len: int, u, delta, A, B, C, Dskip, z,
                  delta_bias, h0, dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                  workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_bwd_varlen(_ref(desc), cu_seqlens, int(total_len), u, delta, A,
                                        B, C, Dskip, z, delta_bias, h0, dy, du, ddelta, dA, dB,
                                        dC, dD, dz, ddelta_bias, dh0, workspace,
                                        workspace_bytes, stream)


def ss_fwd_strided(desc: SsDesc, cu_seqlens, total_len: int, ldb: int, ldc: int, u, delta, A,
                   B, C, Dskip, z, delta_bias, h0, y, last_state, workspace,
                   workspace_bytes: int, stream) -> int:
    return load_library().ss_fwd_strided(_ref(desc), cu_seqlens, int(total_len), int(ldb),
                                         int(ldc), u, delta, A, B, C, Dskip, z, delta_bias, h0,
                                         y, last_state, workspace, workspace_bytes, stream)


def ss_bwd_strided(desc: SsDesc, cu_seqlens, total_len: int, ldb: int, ldc: int, u, delta, A,
                   B, C, Dskip, z, delta_bias, h0, dy, du, ddelta, dA, dB, dC, dD, dz,
                   ddelta_bias, dh0, workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_bwd_strided(_ref(desc), cu_seqlens, int(total_len), int(ldb),
                                         int(ldc), u, delta, A, B, C, Dskip, z, delta_bias, h0,
                                         dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0,
                                         workspace, workspace_bytes, stream)


def ss_workspace_size_complex(desc: SsDesc, backward: int) -> int:
    return load_library().ss_workspace_size_complex(_ref(desc), int(backward))


def ss_fwd_complex(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, h0, y, last_state,
                   workspace, workspace_bytes: int, stream) -> int:
    return load_library().ss_fwd_complex(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias,
                                         h0, y, last_state, workspace, workspace_bytes, stream)


def ss_bwd_complex(desc: SsDesc, u, delta, A, B, C, Dskip, z, delta_bias, h0, dy, du, ddelta,
                   dA, dB, dC, dD, dz, ddelta_bias, dh0, workspace, workspace_bytes: int,
                   stream) -> int:
    return load_library().ss_bwd_complex(_ref(desc), u, delta, A, B, C, Dskip, z, delta_bias,
                                         h0, dy, du, ddelta, dA, dB, dC, dD, dz, ddelta_bias,
                                         dh0, workspace, workspace_bytes, stream)


def ss_plan_query(desc: SsDesc, backward: int, out: SsPlan) -> int:
    return load_library().ss_plan_query(_ref(desc), int(backward), _ref(out))


def ss_status_string(status: int) -> str:
    return load_library().ss_status_string(int(status)).decode()


def ss_last_error() -> str:
    return load_library().ss_last_error().decode()


# ------------------------------------------------------------- tensor helpers

def _raise(status: int, who: str):
    msg = f"{who}: {ss_status_string(status)}: {ss_last_error()}"
    if status == SS_ERR_INVALID_PROBLEM:
        raise ValueError(msg)
    if status == SS_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _ptr(t: Optional[torch.Tensor]):
    # (a plain int: ctypes converts it for the c_void_p parameters)
    return None if t is None else t.data_ptr()


def _check(t: Optional[torch.Tensor], name: str, shape, dtype, device, contiguous=True):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.shape != shape:                      # torch.Size compares equal to a tuple
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _row_stride(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> int:
    """Elements between consecutive rows of a [..., N] tensor (B, C, dB, dC)
    whose rows are contiguous and evenly spaced: N when packed, more for a
    column slice of a wider matrix.  0 for None."""
    _check(t, name, shape, dtype, device, contiguous=False)
    if t is None:
        return 0
    N = shape[-1]
    if t.is_contiguous():
        return N
    if N > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    ld, inner = None, 1
    for i in range(len(shape) - 2, -1, -1):
        if shape[i] > 1:
            if ld is None:
                ld = t.stride(i)
            elif t.stride(i) != ld * inner:
                raise ValueError(f"{name}: rows must be evenly spaced")
        inner *= shape[i]
    ld = N if ld is None else ld
    if ld < N:
        raise ValueError(f"{name}: row stride {ld} < {N}")
    return ld


def _rows_like(shape, ld: int, dtype, device) -> torch.Tensor:
    """An output of `shape` [..., N] whose rows lie ld elements apart."""
    N = shape[-1]
    rows = 1
    for x in shape[:-1]:
        rows *= x
    base = torch.empty(max((rows - 1) * ld + N, 0) if rows > 0 else 0, dtype=dtype,
                       device=device)
    strides, inner = [1], ld
    for x in reversed(shape[:-1]):
        strides.insert(0, inner)
        inner *= x
    return base.as_strided(tuple(shape), tuple(strides))


def _desc_for(u: torch.Tensor, A: torch.Tensor, delta_softplus: bool, chunk_len: int) -> SsDesc:
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [B, L, D] and A [D, N]")
    if u.dtype not in _DTYPE_ID or A.dtype not in _DTYPE_ID:
        raise NotImplementedError("dtypes must be float32, float16 or bfloat16")
    Bn, L, D = u.shape
    N = A.shape[1]
    return SsDesc(Bn, L, D, N, 1 if delta_softplus else 0, _DTYPE_ID[u.dtype],
                  _DTYPE_ID[A.dtype], int(chunk_len))


def plan(desc: SsDesc, backward: bool = False) -> SsPlan:
    out = SsPlan()
    st = ss_plan_query(desc, int(backward), out)
    if st != SS_OK:
        _raise(st, "ss_plan_query")
    return out


def workspace_size(desc: SsDesc, backward: bool = False) -> int:
    return ss_workspace_size(desc, int(backward))


def _stream_of(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus: bool = True,
        return_last_state: bool = False, chunk_len: int = 0, y: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, h0: Optional[torch.Tensor] = None,
        last_state: Optional[torch.Tensor] = None
        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Selective-scan forward on the tensors' GPU.

    u, delta, z: [B, L, D]; A: [D, N]; B, C: [B, L, N]; D, delta_bias: [D];
    h0 (state before the first step, zero if None): [B, D, N].
    u / delta / B / C / z share one dtype (f32, f16 or bf16); A / D /
    delta_bias / h0 / last_state are float32 or that dtype.  last_state, if
    given, receives the final state (it may be h0 itself: an in-place state
    update).  Returns (y, last_state or None).
    """
    desc = _desc_for(u, A, delta_softplus, chunk_len)
    dev, io, pa = u.device, u.dtype, A.dtype
    Bn, L, Dd, N = desc.batch, desc.seqlen, desc.dim, desc.dstate
    for t, name, shape, dt in ((u, "u", (Bn, L, Dd), io), (delta, "delta", (Bn, L, Dd), io),
                               (A, "A", (Dd, N), pa), (D, "D", (Dd,), pa),
                               (z, "z", (Bn, L, Dd), io), (delta_bias, "delta_bias", (Dd,), pa)):
        _check(t, name, shape, dt, dev)
    ldb = _row_stride(B, "B", (Bn, L, N), io, dev)
    ldc = _row_stride(C, "C", (Bn, L, N), io, dev)
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    _check(h0, "h0", (Bn, Dd, N), pa, dev)
    _check(last_state, "last_state", (Bn, Dd, N), pa, dev)
    if y is None:
        y = torch.empty((Bn, L, Dd), dtype=io, device=dev)
    _check(y, "y", (Bn, L, Dd), io, dev)
    ls = last_state
    if ls is None and return_last_state:
        ls = torch.empty((Bn, Dd, N), dtype=pa, device=dev)
    need = workspace_size(desc, False)
    if need > 0 and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    if ldb == N and ldc == N:
        who = "ss_fwd_h0" if h0 is not None else "ss_fwd"
        st = ss_fwd_h0(desc, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                       _ptr(delta_bias), _ptr(h0), _ptr(y), _ptr(ls), _ptr(workspace),
                       ws_bytes, _stream_of(dev))
    else:
        who = "ss_fwd_strided"
        st = ss_fwd_strided(desc, None, 0, ldb, ldc, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                            _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(y),
                            _ptr(ls), _ptr(workspace), ws_bytes, _stream_of(dev))
    if st != SS_OK:
        _raise(st, who)
    return y, ls


def _varlen_desc(u, A, cu_seqlens, max_seqlen, delta_softplus, chunk_len) -> SsDesc:
    if u.dim() != 2 or A.dim() != 2:
        raise ValueError("packed u must be [T, D] and A [D, N]")
    if u.dtype not in _DTYPE_ID or A.dtype not in _DTYPE_ID:
        raise NotImplementedError("dtypes must be float32, float16 or bfloat16")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of S + 1 offsets")
    if cu_seqlens.device != u.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous on the tensors' device")
    return SsDesc(cu_seqlens.numel() - 1, int(max_seqlen), u.shape[1], A.shape[1],
                  1 if delta_softplus else 0, _DTYPE_ID[u.dtype], _DTYPE_ID[A.dtype],
                  int(chunk_len))


def fwd_varlen(u, delta, A, B, C, cu_seqlens, max_seqlen: int, D=None, z=None,
               delta_bias=None, delta_softplus: bool = True, h0=None,
               return_last_state: bool = False, chunk_len: int = 0,
               y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               last_state: Optional[torch.Tensor] = None
               ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward over packed variable-length sequences.

    u, delta, z: [T, D]; B, C: [T, N]; cu_seqlens: int32 [S + 1] row offsets
    on the device; max_seqlen >= every sequence's length; h0 / last_state:
    [S, D, N].  Returns (y [T, D], last_state or None).
    """
    desc = _varlen_desc(u, A, cu_seqlens, max_seqlen, delta_softplus, chunk_len)
    dev, io, pa = u.device, u.dtype, A.dtype
    S, Dd, N = desc.batch, desc.dim, desc.dstate
    T = u.shape[0]
    for t, name, shape, dt in ((u, "u", (T, Dd), io), (delta, "delta", (T, Dd), io),
                               (A, "A", (Dd, N), pa), (D, "D", (Dd,), pa),
                               (z, "z", (T, Dd), io), (delta_bias, "delta_bias", (Dd,), pa),
                               (h0, "h0", (S, Dd, N), pa),
                               (last_state, "last_state", (S, Dd, N), pa)):
        _check(t, name, shape, dt, dev)
    ldb = _row_stride(B, "B", (T, N), io, dev)
    ldc = _row_stride(C, "C", (T, N), io, dev)
    if y is None:
        y = torch.empty((T, Dd), dtype=io, device=dev)
    _check(y, "y", (T, Dd), io, dev)
    ls = last_state
    if ls is None and return_last_state:
        ls = torch.empty((S, Dd, N), dtype=pa, device=dev)
    need = workspace_size(desc, False)
    if need > 0 and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel()
    if ldb == N and ldc == N:
        who = "ss_fwd_varlen"
        st = ss_fwd_varlen(desc, _ptr(cu_seqlens), T, _ptr(u), _ptr(delta), _ptr(A), _ptr(B),
                           _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0), _ptr(y),
                           _ptr(ls), _ptr(workspace), ws_bytes, _stream_of(dev))
    else:
        who = "ss_fwd_strided"
        st = ss_fwd_strided(desc, _ptr(cu_seqlens), T, ldb, ldc, _ptr(u), _ptr(delta), _ptr(A),
                            _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), _ptr(h0),
                            _ptr(y), _ptr(ls), _ptr(workspace), ws_bytes, _stream_of(dev))
    if st != SS_OK:
        _raise(st, who)
    return y, ls


def _pairs(t: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """A complex tensor as its (re, im) float pairs (a view); float tensors
    with a trailing axis of 2 pass through."""
    if t is None or not t.is_complex():
        return t
    return torch.view_as_real(t)


def _complex_desc(u, A, delta_softplus, chunk_len) -> SsDesc:
    if u.dim() != 3 or A.dim() != 3 or A.shape[-1] != 2:
        raise ValueError("u must be [B, L, D] and A [D, N, 2] (re, im pairs) or complex [D, N]")
    if u.dtype not in _DTYPE_ID or A.dtype not in _DTYPE_ID:
        raise NotImplementedError("dtypes must be float32, float16 or bfloat16 (pairs)")
    Bn, L, D = u.shape
    return SsDesc(Bn, L, D, A.shape[1], 1 if delta_softplus else 0, _DTYPE_ID[u.dtype],
                  _DTYPE_ID[A.dtype], int(chunk_len))


def fwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                delta_softplus: bool = True, h0=None, return_last_state: bool = False,
                chunk_len: int = 0, last_state: Optional[torch.Tensor] = None
                ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Complex-valued forward: A [D, N], B / C [B, L, N], h0 / last_state
    [B, D, N] complex, given either as torch complex64 tensors or as float
    tensors with a trailing (re, im) axis of 2; everything else as ``fwd``.
    Returns (y [B, L, D] real, last_state as (re, im) pairs or None)."""
    A, B, C, h0, last_state = (_pairs(t) for t in (A, B, C, h0, last_state))
    desc = _complex_desc(u, A, delta_softplus, chunk_len)
    dev, io, pa = u.device, u.dtype, A.dtype
    Bn, L, Dd, N = desc.batch, desc.seqlen, desc.dim, desc.dstate
    for t, name, shape, dt in ((u, "u", (Bn, L, Dd), io), (delta, "delta", (Bn, L, Dd), io),
                               (A, "A", (Dd, N, 2), pa), (B, "B", (Bn, L, N, 2), io),
                               (C, "C", (Bn, L, N, 2), io), (D, "D", (Dd,), pa),
                               (z, "z", (Bn, L, Dd), io), (delta_bias, "delta_bias", (Dd,), pa),
                               (h0, "h0", (Bn, Dd, N, 2), pa),
                               (last_state, "last_state", (Bn, Dd, N, 2), pa)):
        _check(t, name, shape, dt, dev)
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    y = torch.empty((Bn, L, Dd), dtype=io, device=dev)
    ls = last_state
    if ls is None and return_last_state:
        ls = torch.empty((Bn, Dd, N, 2), dtype=pa, device=dev)
    need = ss_workspace_size_complex(desc, 0)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need > 0 else None
    st = ss_fwd_complex(desc, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                        _ptr(delta_bias), _ptr(h0), _ptr(y), _ptr(ls), _ptr(ws), need,
                        _stream_of(dev))
    if st != SS_OK:
        _raise(st, "ss_fwd_complex")
    return y, ls


def bwd_complex(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None,
                delta_softplus: bool = True, h0=None, chunk_len: int = 0
                ) -> Dict[str, Optional[torch.Tensor]]:
    """Backward of ``fwd_complex`` for sum(dy * y): the dict of ``bwd`` with
    dA / dB / dC / dh0 as (dL/dRe, dL/dIm) pairs in the layouts of A / B /
    C / h0 (float pairs)."""
    A, B, C, h0 = (_pairs(t) for t in (A, B, C, h0))
    desc = _complex_desc(u, A, delta_softplus, chunk_len)
    dev, io, pa = u.device, u.dtype, A.dtype
    Bn, L, Dd, N = desc.batch, desc.seqlen, desc.dim, desc.dstate
    for t, name, shape, dt in ((u, "u", (Bn, L, Dd), io), (delta, "delta", (Bn, L, Dd), io),
                               (A, "A", (Dd, N, 2), pa), (B, "B", (Bn, L, N, 2), io),
                               (C, "C", (Bn, L, N, 2), io), (D, "D", (Dd,), pa),
                               (z, "z", (Bn, L, Dd), io), (delta_bias, "delta_bias", (Dd,), pa),
                               (dy, "dy", (Bn, L, Dd), io), (h0, "h0", (Bn, Dd, N, 2), pa)):
        _check(t, name, shape, dt, dev)
    if dy is None:
        raise ValueError("dy is required")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    out = {
        "du": torch.empty((Bn, L, Dd), dtype=io, device=dev),
        "ddelta": torch.empty((Bn, L, Dd), dtype=io, device=dev),
        "dA": torch.empty((Dd, N, 2), dtype=pa, device=dev),
        "dB": torch.empty((Bn, L, N, 2), dtype=io, device=dev),
        "dC": torch.empty((Bn, L, N, 2), dtype=io, device=dev),
        "dD": torch.empty((Dd,), dtype=pa, device=dev) if D is not None else None,
        "dz": torch.empty((Bn, L, Dd), dtype=io, device=dev) if z is not None else None,
        "ddelta_bias": torch.empty((Dd,), dtype=pa, device=dev) if delta_bias is not None else None,
        "dh0": torch.empty((Bn, Dd, N, 2), dtype=pa, device=dev) if h0 is not None else None,
    }
    need = ss_workspace_size_complex(desc, 1)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = ss_bwd_complex(desc, _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                        _ptr(delta_bias), _ptr(h0), _ptr(dy), _ptr(out["du"]),
                        _ptr(out["ddelta"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                        _ptr(out["dD"]), _ptr(out["dz"]), _ptr(out["ddelta_bias"]),
                        _ptr(out["dh0"]), _ptr(ws), ws.numel(), _stream_of(dev))
    if st != SS_OK:
        _raise(st, "ss_bwd_complex")
    return out


def decode_step(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                delta_softplus: bool = True) -> torch.Tensor:
    """One recurrence step on a carried state, updated in place.

    state: [B, D, N] (param dtype); u, delta, z: [B, D]; B, C: [B, N].
    Returns y: [B, D].
    """
    y, _ = fwd(u.unsqueeze(1), delta.unsqueeze(1), A, B.unsqueeze(1), C.unsqueeze(1), D,
               None if z is None else z.unsqueeze(1), delta_bias, delta_softplus,
               h0=state, last_state=state)
    return y.squeeze(1)


def _bwd_call(desc, cu_seqlens, row_shape, state_shape, u, delta, A, B, C, D, z, delta_bias,
              dy, h0, workspace, dB, dC, who_packed):
    """Shared body of ``bwd`` / ``bwd_varlen``: row_shape is (B, L) or (T,)."""
    dev, io, pa = u.device, u.dtype, A.dtype
    Dd, N = desc.dim, desc.dstate
    rd, rn = tuple(row_shape) + (Dd,), tuple(row_shape) + (N,)
    for t, name, shape, dt in ((u, "u", rd, io), (delta, "delta", rd, io),
                               (A, "A", (Dd, N), pa), (D, "D", (Dd,), pa),
                               (z, "z", rd, io), (delta_bias, "delta_bias", (Dd,), pa),
                               (dy, "dy", rd, io), (h0, "h0", state_shape, pa)):
        _check(t, name, shape, dt, dev)
    ldb = _row_stride(B, "B", rn, io, dev)
    ldc = _row_stride(C, "C", rn, io, dev)
    if dy is None:
        raise ValueError("dy is required")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU")
    # dB / dC: given outputs must share B's / C's row stride; new ones get it
    if dB is None:
        dB = _rows_like(rn, ldb, io, dev)
    if dC is None:
        dC = _rows_like(rn, ldc, io, dev)
    if _row_stride(dB, "dB", rn, io, dev) != ldb or _row_stride(dC, "dC", rn, io, dev) != ldc:
        raise ValueError("dB / dC must have the row strides of B / C")
    out = {
        "du": torch.empty(rd, dtype=io, device=dev),
        "ddelta": torch.empty(rd, dtype=io, device=dev),
        "dA": torch.empty((Dd, N), dtype=pa, device=dev),
        "dB": dB, "dC": dC,
        "dD": torch.empty((Dd,), dtype=pa, device=dev) if D is not None else None,
        "dz": torch.empty(rd, dtype=io, device=dev) if z is not None else None,
        "ddelta_bias": torch.empty((Dd,), dtype=pa, device=dev) if delta_bias is not None else None,
        "dh0": torch.empty(state_shape, dtype=pa, device=dev) if h0 is not None else None,
    }
    need = workspace_size(desc, True)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ptrs = [_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
            _ptr(delta_bias), _ptr(h0), _ptr(dy), _ptr(out["du"]), _ptr(out["ddelta"]),
            _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
            _ptr(out["dz"]), _ptr(out["ddelta_bias"]), _ptr(out["dh0"]), _ptr(workspace),
            workspace.numel(), _stream_of(dev)]
    T = 1
    for x in row_shape:
        T *= x
    if ldb != N or ldc != N:
        who = "ss_bwd_strided"
        st = ss_bwd_strided(desc, _ptr(cu_seqlens), T if cu_seqlens is not None else 0, ldb,
                            ldc, *ptrs)
    elif cu_seqlens is not None:
        who = who_packed
        st = ss_bwd_varlen(desc, _ptr(cu_seqlens), T, *ptrs)
    else:
        who = who_packed
        st = ss_bwd_h0(desc, *ptrs)
    if st != SS_OK:
        _raise(st, who)
    return out


def bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, dy=None,
        delta_softplus: bool = True, chunk_len: int = 0,
        workspace: Optional[torch.Tensor] = None,
        h0: Optional[torch.Tensor] = None, dB: Optional[torch.Tensor] = None,
        dC: Optional[torch.Tensor] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Selective-scan backward: gradients of sum(dy * y).

    Returns a dict with du, ddelta, dA, dB, dC, dD, dz, ddelta_bias, dh0
    (dD / dz / ddelta_bias / dh0 are None when D / z / delta_bias / h0 are
    None).  dB / dC, if given, are written in place and must have the row
    strides of B / C (for column slices of a wider matrix, only those
    columns are written); new ones are allocated with those strides.
    """
    desc = _desc_for(u, A, delta_softplus, chunk_len)
    return _bwd_call(desc, None, (desc.batch, desc.seqlen), (desc.batch, desc.dim, desc.dstate),
                     u, delta, A, B, C, D, z, delta_bias, dy, h0, workspace, dB, dC,
                     "ss_bwd_h0" if h0 is not None else "ss_bwd")


def bwd_varlen(u, delta, A, B, C, cu_seqlens, max_seqlen: int, D=None, z=None,
               delta_bias=None, dy=None, delta_softplus: bool = True, h0=None,
               chunk_len: int = 0, workspace: Optional[torch.Tensor] = None,
               dB: Optional[torch.Tensor] = None, dC: Optional[torch.Tensor] = None
               ) -> Dict[str, Optional[torch.Tensor]]:
    """Backward of ``fwd_varlen``: gradients of sum(dy * y) over the packed rows.

    Shapes as ``fwd_varlen`` (dy: [T, D]); returns the dict of ``bwd`` with
    du / ddelta / dz [T, D], dB / dC [T, N] and dh0 [S, D, N].  Rows that no
    sequence covers get unspecified gradients.
    """
    desc = _varlen_desc(u, A, cu_seqlens, max_seqlen, delta_softplus, chunk_len)
    return _bwd_call(desc, cu_seqlens, (u.shape[0],), (desc.batch, desc.dim, desc.dstate),
                     u, delta, A, B, C, D, z, delta_bias, dy, h0, workspace, dB, dC,
                     "ss_bwd_varlen")


class _SelectiveScanFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0):
        y, _ = fwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0=h0)
        ctx.delta_softplus = delta_softplus
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, h0)
        return y

    @staticmethod
    def backward(ctx, dy):
        u, delta, A, B, C, D, z, delta_bias, h0 = ctx.saved_tensors
        g = bwd(u, delta, A, B, C, D, z, delta_bias, dy.contiguous(), ctx.delta_softplus,
                h0=h0)
        return (g["du"], g["ddelta"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"],
                g["ddelta_bias"], None, g["dh0"])


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus: bool = True, h0=None) -> torch.Tensor:
    """Differentiable forward (autograd backward runs ``ss_bwd_h0``)."""
    return _SelectiveScanFn.apply(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0)
