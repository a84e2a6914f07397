"""Build libss.so (the HIP selective-scan library) for gfx950.

    python -m mamba_selective_scan_02_amd.build

Every source is compiled with hipcc for gfx950 only; the objects go to
``_build/`` at the repository root and the library to
``mamba_selective_scan_02_amd/libss.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libss.so")
# (source, object name, extra flags): ss_fwd_scan.hip is compiled once per I/O
# type so that its instantiations build in parallel.
SOURCES = [("ss_api.cpp", "ss_api", []), ("ss_fwd.hip", "ss_fwd", []),
           ("ss_fwd_scan.hip", "ss_fwd_scan_f32", ["-DSS_SCAN_IO=0"]),
           ("ss_fwd_scan.hip", "ss_fwd_scan_f16", ["-DSS_SCAN_IO=1"]),
           ("ss_fwd_scan.hip", "ss_fwd_scan_bf16", ["-DSS_SCAN_IO=2"]),
           ("ss_fwd_tile.hip", "ss_fwd_tile", []), ("ss_bwd.hip", "ss_bwd", []),
           ("ss_bwd_tile.hip", "ss_bwd_tile", []), ("ss_cplx.hip", "ss_cplx", [])]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are disabled: the compiler would otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result", "-Wno-unknown-pragmas",
          "-I" + os.path.join(ROOT, "include")]


def _compile(entry, verbose: bool) -> str:
    src, name, flags = entry
    obj = os.path.join(BUILD, name + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + COMMON + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_microbench(verbose: bool = False) -> str:
    """Hardware-rate microbenchmark (microbench/rates.hip -> microbench/rates)."""
    src = os.path.join(PKG, "microbench", "rates.hip")
    out = os.path.join(PKG, "microbench", "rates")
    cmd = [HIPCC, "-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-Wno-unused-result", src, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("microbench build failed:\n" + r.stdout + r.stderr)
    return out


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
    build_microbench(verbose="-q" not in sys.argv)
