"""The bulk append's division-free rounding rule, checked on the CPU against IEEE division.

The kernel computes INT8 and 4-bit codes as rint(x * fl(1/s)) and falls back to
rint(fl(x / s)) only where the product lies within 2^-15 of a half-integer; the rule is
exact for quotients below 128.  tests/native/rint_quotient.c restates it in plain C and
compares it with the division on random fp16 scales and values, half of them placed a few
ulps around the rounding boundaries.  (The GPU parity tests compare every appended pool
with the oracle's byte for byte.)
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_reciprocal_rounding_matches_division(tmp_path):
    exe = tmp_path / "rint_quotient"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                    os.path.join(ROOT, "tests", "native", "rint_quotient.c"), "-lm"], check=True)
    r = subprocess.run([str(exe), "20000000"], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " mismatches 0 (fused 0)" in r.stdout
