"""The kernels divide by an inner scale with a two-term binary32 reciprocal
from a per-code table (one multiply and one or two fmas), not a division.
tests/pins/inner_quotient_check.c checks, on the CPU, that this gives the
correctly rounded quotient (RNE path) and the exact fixed-point input of the
stochastic-rounding convert (SR path, with and without the clamp) for every
scale code of E4M3 and UE5M3.  It restates the kernels' arithmetic, not the
oracle's; the oracle divides."""
import os
import subprocess
import tempfile

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pins", "inner_quotient_check.c")


def test_two_term_inner_quotients_are_exact():
    d = tempfile.mkdtemp(prefix="fp4q")
    exe = os.path.join(d, "inner_quotient_check")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", SRC, "-o", exe, "-lm"], check=True)
    # a tenth of the full sample (the full run, argument 1, checks 3.2e8 values)
    r = subprocess.run([exe, "0.1"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout, r.stdout
