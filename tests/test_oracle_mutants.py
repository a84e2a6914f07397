"""The oracle's pins must catch plausible mistakes (CPU only).

Each case copies the oracle's C source, plants one mistake in the copy (a
dropped term, a wrong sign, a wrong index, a transposed operand, a missing
factor in the backward), builds it into a temporary library and runs the pin
suite (tests/test_oracle_pins.py) against it through SS_ORACLE_LIB.  The suite
must fail for every mutant.  Each mutant is also planted in the float
instantiation alone (the single-precision build behind fwd_f32 / bwd_f32),
which the suite must catch through its float-build pins.  The oracle source
itself is never modified.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

# (name, exact text in ss_oracle_impl.h, replacement, occurrence to replace:
#  0 = forward channel loop, 1 = forward pass inside the backward, None = all)
MUTANTS = [
    ("bias dropped", "REAL x = delta[i] + (bias ? bias[d] : (REAL)0);", "REAL x = delta[i];", 0),
    ("softplus sign", "return (REAL)log1p(exp((double)x));", "return (REAL)log1p(exp(-(double)x));", None),
    ("decay dropped", "h[n] = a * h[n] + dl * Bt[n] * u[i];", "h[n] = h[n] + dl * Bt[n] * u[i];", 0),
    ("delta dropped from input", "h[n] = a * h[n] + dl * Bt[n] * u[i];", "h[n] = a * h[n] + Bt[n] * u[i];", 0),
    ("A transposed", "REAL a = (REAL)exp((double)(dl * A[d * N + n]));  /* A is [D, N] */",
     "REAL a = (REAL)exp((double)(dl * A[n * D + d]));", 0),
    ("B batch offset dropped", "const REAL* Bt = Bm + (b * L + t) * N;             /* [B, L, N] */",
     "const REAL* Bt = Bm + t * N;", 0),
    ("C uses B", "o += Ct[n] * h[n];", "o += Bt[n] * h[n];", 0),
    ("readout before update", "h[n] = a * h[n] + dl * Bt[n] * u[i];\n      o += Ct[n] * h[n];",
     "o += Ct[n] * h[n];\n      h[n] = a * h[n] + dl * Bt[n] * u[i];", 0),
    ("skip index", "if (Dskip) o += Dskip[d] * u[i];\n    if (z)", "if (Dskip) o += Dskip[0] * u[i];\n    if (z)", 0),
    ("gate without z", "if (z) o = o * z[i] * FN(sigmoid)(z[i]);", "if (z) o = o * FN(sigmoid)(z[i]);", 0),
    ("adjoint decay dropped", "dh[n] *= a;", "dh[n] *= (REAL)1;", None),
    ("dz sign", "((REAL)1 + z[i] * ((REAL)1 - s))", "((REAL)1 - z[i] * ((REAL)1 - s))", None),
    ("dA uses current state", "const REAL ga = dh[n] * hprev;", "const REAL ga = dh[n] * hcur;", None),
    ("dB uses gate grad", "dB_part[(b * L + t) * N + n] += dh[n] * dls[t] * u[i];",
     "dB_part[(b * L + t) * N + n] += g * dls[t] * u[i];", None),
    ("softplus backward dropped", "REAL dx = p->delta_softplus ? ddl * FN(sigmoid)(xs[t]) : ddl;",
     "REAL dx = ddl;", None),
    ("du skip term dropped", "REAL dui = Dskip ? g * Dskip[d] : (REAL)0;", "REAL dui = 0;", None),
    ("dC uses previous state", "dC_part[(b * L + t) * N + n] += g * hcur;",
     "dC_part[(b * L + t) * N + n] += g * hprev;", None),
    ("h0 ignored in forward", "h[n] = h0_row ? h0_row[n] : 0;", "h[n] = 0;", None),
    ("h0 ignored in backward recompute", "hist[n] = h0 ? h0[(b * D + d) * N + n] : 0;",
     "hist[n] = 0;", None),
    ("dh0 without the first decay", "dh0[(b * D + d) * N + n] = dh[n];",
     "dh0[(b * D + d) * N + n] = dh[n] / ahist[n];", None),
]


def _mutate(text, old, new, occ):
    assert old in text, old
    if occ is None:
        return text.replace(old, new)
    parts = text.split(old)
    assert len(parts) > occ + 1, (old, occ)
    return old.join(parts[:occ + 1]) + new + old.join(parts[occ + 1:])


def _run_mutant(case, tmp, f32_only=False):
    """Build the mutant and run the pins against it.  f32_only plants the
    mistake in the float instantiation alone (fwd_f32 / bwd_f32), leaving the
    double one intact: the pins must then catch it through the float build."""
    name, old, new, occ = case
    d = os.path.join(tmp, ("f32_" if f32_only else "") + name.replace(" ", "_"))
    os.makedirs(d)
    with open(os.path.join(ORACLE, "ss_oracle_impl.h")) as f:
        text = f.read()
    with open(os.path.join(ORACLE, "ss_oracle.c")) as f:
        csrc = f.read()
    if f32_only:
        inc = '#include "ss_oracle_impl.h"'
        assert csrc.count(inc) == 2, "expected the double and the float instantiation"
        first = csrc.index(inc) + len(inc)
        csrc = csrc[:first] + csrc[first:].replace(inc, '#include "ss_oracle_impl_f32.h"')
        with open(os.path.join(d, "ss_oracle_impl.h"), "w") as f:
            f.write(text)
        with open(os.path.join(d, "ss_oracle_impl_f32.h"), "w") as f:
            f.write(_mutate(text, old, new, occ))
    else:
        with open(os.path.join(d, "ss_oracle_impl.h"), "w") as f:
            f.write(_mutate(text, old, new, occ))
    with open(os.path.join(d, "ss_oracle.c"), "w") as f:
        f.write(csrc)
    lib = os.path.join(d, "libmut.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-ffp-contract=off", os.path.join(d, "ss_oracle.c"), "-o", lib, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, SS_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


@pytest.mark.parametrize("f32_only", [False, True], ids=["both_builds", "float_build_only"])
def test_pins_catch_every_mutant(f32_only):
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda c: _run_mutant(c, tmp, f32_only), MUTANTS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"pins did not catch: {survivors}"
