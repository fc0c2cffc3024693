"""Mutation test of the oracle's pins.

Each case copies ``oracle/`` to a temporary directory, plants one plausible
mistake in the copy (a swapped index, a wrong rounding mode, a loosened
tolerance input, ...) and runs ``tests/test_oracle_pins.py`` against that
copy (the ``MNB_ORACLE_ROOT`` hook of ``tests/conftest.py``).  Every mutant
must fail at least one pin; the unchanged copy and an equivalent rewrite must
pass.  The mistakes are planted on the CPU only; no GPU is involved.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
C_SRC = "mnb_oracle.c"
PY_SRC = "__init__.py"

# (name, file, text in the oracle, replacement)
MUTANTS = [
    ("nibble_order_swapped", C_SRC,
     "return (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "return (k % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    ("zero_point_order_swapped", C_SRC,
     "return (b % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
     "return (b % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    ("zero_point_not_subtracted", C_SRC,
     "double w = (double)(q - z) * s;", "double w = (double)q * s;"),
    ("explicit_zero_point_ignored", C_SRC,
     "double w = (double)(q - z) * s;", "double w = (double)(q - 8) * s;"),
    ("default_zero_point_7", C_SRC,
     "if (zp == NULL) return 8;", "if (zp == NULL) return 7;"),
    ("scale_blocks_reversed", C_SRC,
     "scales[n * nblocks + b]", "scales[n * nblocks + (nblocks - 1 - b)]"),
    ("block_size_64", C_SRC,
     "int64_t b = k / 32;", "int64_t b = k / 64;"),
    ("row_stride_ignored", C_SRC,
     "double p = a[r * K + k] * w;", "double p = a[k] * w;"),
    ("bf16_activations_not_rounded", C_SRC,
     "a[i] = mnb_oracle_f16_to_f64(h);",
     "a[i] = a_is_bf16 ? mnb_oracle_bf16_to_f64(A_bits[i]) : mnb_oracle_f16_to_f64(h);"),
    ("single_rounding_to_bf16", C_SRC,
     "if (y_bf16) y_bf16[o] = mnb_oracle_f16_to_bf16(h);",
     "if (y_bf16) y_bf16[o] = f64_to_bf16(sum);"),
    ("ties_away_from_zero", C_SRC,
     "if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;",
     "if (frac >= 0.5) n += 1.0;"),
    ("subnormals_flushed", C_SRC,
     "if (e < emin) e = emin;", "if (e < emin) return copysign(0.0, x);"),
    ("no_overflow_to_infinity", C_SRC,
     "if (isinf(v) || av > maxfinite) return sbit | (expall << (p - 1));",
     "if (isinf(v)) return sbit | (expall << (p - 1));\n"
     "    if (av > maxfinite) av = maxfinite;"),
    ("weights_f16_ignored", C_SRC,
     "if (weights_f16) w = ", "if (0) w = "),
    ("abs_sum_tripled", C_SRC,
     "asum += fabs(p);", "asum += 3.0 * fabs(p);"),
    ("abs_sum_signed", C_SRC,
     "asum += fabs(p);", "asum += p;"),
    ("abs_sum_of_activations", C_SRC,
     "asum += fabs(p);", "asum += fabs(a[r * K + k]);"),
    ("ulp_sixteen_times", PY_SRC,
     "ulp = np.ldexp(1.0, e - 10)", "ulp = np.ldexp(1.0, e - 6)"),
    ("ulp_half", PY_SRC,
     "ulp = np.ldexp(1.0, e - 10)", "ulp = np.ldexp(1.0, e - 11)"),
    ("ulp_subnormal_floor", PY_SRC,
     "e = np.maximum(expo - 15, -14)", "e = np.maximum(expo - 15, -15)"),
    ("ulp_finite_at_infinity", PY_SRC,
     "return np.where(expo == 31, np.inf, ulp)", "return ulp"),
]

# Rewrites that must keep every pin green (the harness itself is sound).
EQUIVALENT = [
    ("unchanged", C_SRC, None, None),
    ("factors_commuted", C_SRC,
     "double w = (double)(q - z) * s;", "double w = s * (double)(q - z);"),
]


def _run_pins(tmp, name, fname, old, new):
    root = os.path.join(tmp, name)
    dst = os.path.join(root, "oracle")
    shutil.copytree(ORACLE, dst, ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    if old is not None:
        path = os.path.join(dst, fname)
        with open(path) as f:
            text = f.read()
        assert text.count(old) == 1, "mutation site of %s not found exactly once" % name
        with open(path, "w") as f:
            f.write(text.replace(old, new))
    env = dict(os.environ, MNB_ORACLE_ROOT=root, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py")]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return p.returncode, p.stdout[-2000:] + p.stderr[-2000:]


def _run_all(cases, tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        futs = {c[0]: ex.submit(_run_pins, str(tmp_path), *c) for c in cases}
        return {k: f.result() for k, f in futs.items()}


def test_every_mutant_fails_a_pin(tmp_path):
    res = _run_all(MUTANTS, tmp_path)
    survivors = [k for k, (rc, _) in res.items() if rc != 1]
    # pytest exits 1 when a test failed; anything else (2: collection error,
    # 0: all passed) means the mutant was not caught by a pin.
    assert not survivors, {k: res[k][1] for k in survivors}


def test_equivalent_rewrites_pass(tmp_path):
    res = _run_all(EQUIVALENT, tmp_path)
    bad = {k: out for k, (rc, out) in res.items() if rc != 0}
    assert not bad, bad


@pytest.mark.parametrize("name,fname,old,new", MUTANTS + EQUIVALENT[1:],
                         ids=[m[0] for m in MUTANTS + EQUIVALENT[1:]])
def test_mutation_site_exists(name, fname, old, new):
    with open(os.path.join(ORACLE, fname)) as f:
        assert f.read().count(old) == 1, name
