"""The hardware rounding rules the quantize-append kernels rely on, checked
exhaustively on the GPU by the standalone probe tests/probes/rounding_rules
(compiled by build()): the FP8 conversion instructions against encoding by
exponent and mantissa, the hardware reciprocal plus one Newton step against
the correctly rounded reciprocal (every significand at exponents -40..20),
and the correction step with RN(1/qmax) against the correctly rounded
division (every fp32 range value in [1e-8, 2^17])."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "rounding_rules")
CHECKS = ["fp8_e4m3", "fp8_e5m2", "recip_newton", "div_qmax_3", "div_qmax_15", "div_qmax_127", "div_qmax_255"]


def test_rounding_rules_hold_on_every_input():
    assert os.path.exists(PROBE), "tests/probes/rounding_rules is built by __graft_entry__.build()"
    r = subprocess.run([PROBE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    counts = {}
    for line in r.stdout.splitlines():
        if ": mismatches " in line:
            name, n = line.split(": mismatches ")
            counts[name] = int(n)
    assert sorted(counts) == sorted(CHECKS), r.stdout
    assert all(v == 0 for v in counts.values()), r.stdout
