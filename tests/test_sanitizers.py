"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host code (CPU only).

Two pieces of host code run on every call and are checked here:

* the CPU oracle (oracle/ss_oracle.c), rebuilt with gcc -fsanitize=address,undefined
  and run under the whole pin suite (tests/test_oracle_pins.py);
* the library's host side (csrc/ss_api.cpp: descriptor, pointer and workspace
  validation, planning, the static-scratch lookup), rebuilt with the host pass
  of hipcc sanitized (device code is untouched) and linked with the normal
  objects of the other sources, then run under the C-ABI host tests
  (tests/test_abi_host.py), which make validation-only calls.

The interpreter itself is not instrumented, so the sanitizer runtime is
preloaded into the test's subprocess.  A negative control per runtime (a heap
overflow in a throwaway library) shows that the setup reports errors.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "mamba_selective_scan_02_amd", "csrc")
OBJS = os.path.join(ROOT, "_build")

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
           "PYTHONDONTWRITEBYTECODE": "1"}


def _gcc_asan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(cmd, preload, extra_env=None, timeout=600):
    env = dict(os.environ, **SAN_ENV, LD_PRELOAD=preload, **(extra_env or {}))
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


OVERFLOW_C = r"""
#include <stdlib.h>
int overflow(int n) {
  int* p = (int*)malloc(sizeof(int) * n);
  p[n] = 1;                     /* one past the end */
  int r = p[0];
  free(p);
  return r;
}
"""


def _negative_control(compiler, flags, preload, tmp):
    src = os.path.join(tmp, "ovf.c")
    with open(src, "w") as f:
        f.write(OVERFLOW_C)
    lib = os.path.join(tmp, "libovf.so")
    subprocess.run([compiler, "-shared", "-fPIC", "-g", *flags, src, "-o", lib], check=True,
                   capture_output=True)
    code = f"import ctypes; ctypes.CDLL({lib!r}).overflow(4)"
    r = _run([sys.executable, "-c", code], preload)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_oracle_under_asan_ubsan():
    asan = _gcc_asan()
    if shutil.which("gcc") is None or asan is None:
        pytest.skip("gcc AddressSanitizer runtime not available")
    with tempfile.TemporaryDirectory() as tmp:
        _negative_control("gcc", ["-fsanitize=address"], asan, tmp)
        lib = os.path.join(tmp, "libss_oracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-ffp-contract=off", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                        os.path.join(ROOT, "oracle", "ss_oracle.c"), "-o", lib, "-lm"],
                       check=True, capture_output=True)
        r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                  os.path.join(ROOT, "tests", "test_oracle_pins.py")], asan,
                 {"SS_ORACLE_LIB": lib})
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "passed" in r.stdout


def test_library_host_code_under_asan_ubsan():
    asan = _clang_asan()
    if not os.path.exists(HIPCC) or asan is None:
        pytest.skip("hipcc or its AddressSanitizer runtime not available")
    others = [os.path.join(OBJS, n) for n in os.listdir(OBJS)
              if n.endswith(".o") and n != "ss_api.o"] if os.path.isdir(OBJS) else []
    if len(others) < 8:
        pytest.skip("build the library first (python -m mamba_selective_scan_02_amd.build)")
    clang = os.path.join(asan.split("/lib/clang/")[0], "bin", "clang")   # the same toolchain
    with tempfile.TemporaryDirectory() as tmp:
        if os.path.exists(clang):
            _negative_control(clang, ["-fsanitize=address"], asan, tmp)
        obj = os.path.join(tmp, "ss_api_san.o")
        # host pass only: each sanitizer flag is scoped with -Xarch_host
        host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer"]
        r = subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                            *host_san, "-I" + os.path.join(ROOT, "include"), "-x", "hip", "-c",
                            os.path.join(CSRC, "ss_api.cpp"), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        lib = os.path.join(tmp, "libss_san.so")
        r = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *host_san, obj,
                            *others, "-o", lib], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        r = _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                  os.path.join(ROOT, "tests", "test_abi_host.py")], asan, {"SS_LIBRARY": lib})
        assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
        assert "passed" in r.stdout
