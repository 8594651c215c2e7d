"""The oracle's pins are strong enough: each of ten plausible mistakes,
planted in a modified copy of the oracle's source (never the file the other
tests build), makes tests/test_oracle.py fail.

Each mistake is a text substitution on a copy of oracle/mxfp4_oracle.c: the
original fragment must occur exactly once in the source, so a mutant that no
longer applies fails loudly instead of passing vacuously."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

# name -> (fragment of the oracle's source, the mistaken replacement)
MUTANTS = {
    "scale_rounding_threshold": ("u = (u + 0x00200000u) & 0xFF800000u;",
                                 "u = (u + 0x00400000u) & 0xFF800000u;"),
    "scale_exponent_offset": ("int s = biased - 127 - 2;", "int s = biased - 127 - 1;"),
    "saturation_code": ("code = 7;", "code = 6;"),
    "tie_direction": ("(d == best && (c % 2) == 0)", "(d == best && (c % 2) == 1)"),
    "sign_of_zero_dropped": ("if (signbit(x)) code |= 8;", "if (x < 0) code |= 8;"),
    "nibble_order": ("(uint8_t)(lo | (hi << 4));", "(uint8_t)(hi | (lo << 4));"),
    "transposed_b": ("double p = a[k] * b[k];", "double p = a[k] * b_deq[k * N + n];"),
    "last_k_term_dropped": ("for (int64_t k = 0; k < K; ++k) {\n                double p",
                            "for (int64_t k = 0; k < K - 1; ++k) {\n                double p"),
    "dequant_sign_dropped": ("return (code & 8) ? -v : v;", "return v;"),
    "abs_sum_doubled": ("s += fabs(a_deq[m * K + k] * b_deq[n * K + k]);",
                        "s += 2.0 * fabs(a_deq[m * K + k] * b_deq[n * K + k]);"),
}


def run_pins(lib):
    env = dict(os.environ, MXFP4_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           os.path.join(ROOT, "tests", "test_oracle.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    with open(oracle_build.SRC) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutant %s no longer applies to the oracle source" % name
    mutated = tmp_path / ("mxfp4_oracle_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    lib = oracle_build.build(out=str(tmp_path / "liboracle.so"), src=str(mutated))
    r = run_pins(lib)
    assert r.returncode == 1, "mutant %s survived the pins:\n%s" % (name, r.stdout[-2000:])


def test_unmutated_build_passes(tmp_path):
    lib = oracle_build.build(out=str(tmp_path / "liboracle_plain.so"))
    r = run_pins(lib)
    assert r.returncode == 0, r.stdout[-2000:]
