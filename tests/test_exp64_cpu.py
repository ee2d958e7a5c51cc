"""The float64 exponential of the float64 draw (csrc/sv_exp64.hpp: Tang's
table-driven reduction) built for the host and checked against exact
arithmetic: its 2^(j/256) table against values rederived with 50-digit
decimal arithmetic, and exp64_tab against Decimal.exp on arguments across
the draw's range (a relative error of a few 1e-16 is far inside the 1e-12
band of the float64 draw)."""
import os
import random
import shutil
import subprocess
from decimal import Decimal, getcontext

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_draft_verification_softmax_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include "sv_exp64.hpp"
#include <stdio.h>
int main() {
  for (int j = 0; j < sv::kExp64Table; ++j) printf("%a\n", sv::kExp2Frac[j]);
  double x;
  while (scanf("%la", &x) == 1) printf("%a\n", sv::exp64_tab(x, sv::kExp2Frac));
  return 0;
}
"""


@pytest.fixture(scope="module")
def exp64(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("exp64")
    src, exe = d / "t.cpp", d / "t"
    src.write_text(PROGRAM)
    subprocess.run([HIPCC, "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True,
                   capture_output=True)

    def run(xs):
        inp = "".join(float(x).hex() + "\n" for x in xs)
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True,
                             check=True).stdout.split()
        return [float.fromhex(v) for v in out[:256]], [float.fromhex(v) for v in out[256:]]
    return run


def test_table_is_2_pow_j_over_256_rounded(exp64):
    getcontext().prec = 50
    tab, _ = exp64([])
    ln2 = Decimal(2).ln()
    for j, v in enumerate(tab):
        exact = (Decimal(j) / 256 * ln2).exp()
        assert v == float(exact), (j, v.hex(), float(exact).hex())


def test_relative_error_within_two_ulp(exp64):
    getcontext().prec = 50
    rng = random.Random(7)
    xs = ([rng.uniform(-745.0, 0.0) for _ in range(4000)] +
          [rng.uniform(-40.0, 0.0) for _ in range(8000)] +
          [rng.uniform(-0.02, 0.02) for _ in range(2000)] +
          [0.0, -0.0, -1e-300, -708.3, -700.0, 1.0, 300.0, 709.0] +
          # the reduction's boundaries (n ln2/256 and the midpoints between)
          [float(k) * 0.0027076061740622863 for k in range(-400, 1)] +
          [(k + 0.5) * 0.0027076061740622863 for k in range(-400, 0)])
    _, ys = exp64(xs)
    worst = 0.0
    for x, y in zip(xs, ys):
        e = Decimal(x).exp()
        if e < Decimal(2) ** -1022:
            continue  # subnormal results: absolute error below 2^-1074
        rel = abs((Decimal(y) - e) / e)
        worst = max(worst, float(rel / (Decimal(2) ** -52)))
    assert worst <= 2.0, worst


def test_underflow_and_infinities(exp64):
    _, ys = exp64([float("-inf"), -746.0, -1e300, -800.0])
    assert ys == [0.0, 0.0, 0.0, 0.0]
    _, (y,) = exp64([-745.0])
    assert 0.0 < y < 1e-320  # subnormal, not flushed
