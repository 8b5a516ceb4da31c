"""The bulk append's division-free rounding rule and the E4M3FN encoder, checked on the CPU.

The kernel computes INT8 and 4-bit codes as rint(x * fl(1/s)) and falls back to
rint(fl(x / s)) only where the product lies within 2^-15 of a half-integer; the rule is
exact for quotients below 128.  tests/native/rint_quotient.c restates it in plain C and
compares it with the division on random fp16 scales and values, half of them placed a few
ulps around the rounding boundaries.  FP8 codes keep the division; the library encodes them
with a branch-free closed form, which tests/native/e4m3_encoder.c compares with an encoder
written from the E4M3FN definition over 1.2e8 binary32 patterns.  (The GPU parity tests
compare every appended pool with the oracle's byte for byte.)
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(tmp_path, name, n):
    exe = tmp_path / name
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-o", str(exe),
                    os.path.join(ROOT, "tests", "native", name + ".c"), "-lm"], check=True)
    r = subprocess.run([str(exe), str(n)], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_reciprocal_rounding_matches_division(tmp_path):
    assert " mismatches 0 (fused 0)" in _run(tmp_path, "rint_quotient", 20000000)


def test_e4m3_closed_form_encoder_matches_definition(tmp_path):
    out = _run(tmp_path, "e4m3_encoder", 61).strip()
    assert out.startswith("encoder patterns ") and out.endswith(" mismatches 0"), out
    assert int(out.split()[2]) > 10 ** 8
