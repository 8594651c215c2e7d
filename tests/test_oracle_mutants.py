"""The oracle's pins are strong enough: each of nine plausible mistakes,
planted in a separate build of the oracle (never the one the other tests
use), makes tests/test_oracle.py fail.

Mutants: 1 scale rounding threshold, 2 scale exponent offset, 3 saturation
to the wrong code, 4 tie direction, 5 sign of zero dropped, 6 nibble order swapped,
7 transposed B operand, 8 last K term dropped, 9 sign dropped in
dequantization."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402


@pytest.mark.parametrize("mutant", range(1, 10))
def test_pins_catch_planted_mistake(mutant, tmp_path):
    lib = oracle_build.build(out=str(tmp_path / ("liboracle_m%d.so" % mutant)), mutant=mutant)
    env = dict(os.environ, MXFP4_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, "mutant %d survived the pins:\n%s" % (mutant, r.stdout[-2000:])


def test_unmutated_build_passes(tmp_path):
    lib = oracle_build.build(out=str(tmp_path / "liboracle_m0.so"), mutant=0)
    env = dict(os.environ, MXFP4_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
