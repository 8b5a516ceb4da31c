"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of oracle/kvq_oracle.c (a wrong constant, a
dropped term, a wrong sign, index or operand order), builds it with gcc, and runs the
oracle pin suite against it: the suite must fail.  The unmodified copy must pass.
CPU only; the oracle itself is never modified.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvq_oracle.c")
PINS = ["tests/test_oracle_formats.py", "tests/test_oracle_attention.py", "tests/test_oracle_rk8v4.py",
        "tests/test_oracle_rk4v4.py", "tests/test_oracle_bf16.py"]

# (name, original text, planted mistake)
MUTATIONS = [
    ("int8_divisor_128", "float s32 = a / 127.0f;", "float s32 = a / 128.0f;"),
    ("int8_clamp_128", "if (r < -127.0f) r = -127.0f;", "if (r < -128.0f) r = -128.0f;"),
    ("int8_truncates", "float r = rintf(xg[i] / s);", "float r = truncf(xg[i] / s);"),
    ("int8_unrounded_scale", "float s = orc_f16_to_f32(h);", "float s = s32;"),
    ("fp8_divisor_240", "float s = a / 448.0f;", "float s = a / 240.0f;"),
    ("f16_ties_away", "if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;",
     "if (rest >= 0x1000u) h += 1u;"),
    ("f16_exponent_bias", "v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    ("bf16_fraction_bits", "v = ldexp((double)(128 + m), e - 134);", "v = ldexp((double)(128 + m), e - 135);"),
    ("e4m3_exponent_bias", "v = ldexp((double)(8 + m), e - 10);", "v = ldexp((double)(8 + m), e - 11);"),
    ("e4m3_ties_odd", "pick = (up % 2 == 0) ? up : dn;", "pick = (up % 2 == 1) ? up : dn;"),
    ("k_layout_transposed", "* 256 + (s % 16) * 16 + (d % 16);", "* 256 + (d % 16) * 16 + (s % 16);"),
    ("v_layout_swapped", "(d % 16) * 16 + (s / 16) * 4 + (s % 4);", "(d % 16) * 16 + (s % 4) * 4 + (s / 16);"),
    ("k_scale_index", "if (which == 0) return (((int64_t)r * 4 + j) * (D / 64) + g) * 4 + i;",
     "if (which == 0) return (((int64_t)j * 4 + r) * (D / 64) + g) * 4 + i;"),
    ("gqa_interleaved", "int kvh = h / G;", "int kvh = h % Hkv;"),
    ("causal_bound_dropped", "int last = seq_lens[b] - T + t;", "int last = seq_lens[b] - 1;"),
    ("softmax_scale_dropped", "z[j] = (double)softmax_scale * acc;", "z[j] = acc;"),
    ("no_max_shift", "double w = exp(z[j] - m);\n      l += w;\n      for (int d = 0; d < D; ++d) o[d]",
     "double w = exp(z[j]);\n      l += w;\n      for (int d = 0; d < D; ++d) o[d]"),
    ("dense_unnormalized", "for (int d = 0; d < D; ++d) o[d] /= l;", "for (int d = 0; d < D; ++d) o[d] /= 1.0;"),
    ("paged_v_read_as_k", "row[d] += w * orc_dequant(p, 1, block, kvh, j % 64, d);",
     "row[d] += w * orc_dequant(p, 0, block, kvh, j % 64, d);"),
    ("append_slot_index", "int slot = (int)(pos % 64);", "int slot = (int)((pos + 1) % 64);"),
    ("rk8v4_rotation_norm", "y[j] = (float)(acc / 8.0);", "y[j] = (float)(acc / 64.0);"),
    ("rk8v4_rotation_sign", "acc += odd ? -(double)x[i] : (double)x[i];", "acc += odd ? (double)x[i] : -(double)x[i];"),
    ("rk8v4_query_not_rotated", "for (int d = 0; d < D; ++d) qd[d] = row[d];", "for (int d = 0; d < D; ++d) (void)row[d];"),
    ("int4_divisor_8", "uint16_t h = orc_f32_to_f16_rne(a / 7.0f);", "uint16_t h = orc_f32_to_f16_rne(a / 8.0f);"),
    ("v4_nibble_order", "return word * 8 + 16 * (k % 2) + 4 * (k / 2);", "return word * 8 + 4 * k;"),
    ("v4_scale_group_64", "orc_scale_elem(p->format, 1, slot, d / 32, D)", "orc_scale_elem(p->format, 1, slot, d / 64, D)"),
    ("lloyd_threshold_not_midpoint", "for (int i = 1; i < 16; ++i) t[i] = 0.5 * (L[i - 1] + L[i]);",
     "for (int i = 1; i < 16; ++i) t[i] = 0.4 * L[i - 1] + 0.6 * L[i];"),
    ("rk4_codes_truncated", "codes[i] = (int8_t)rint(127.0 * L[i] / L[15]);", "codes[i] = (int8_t)(127.0 * L[i] / L[15]);"),
    ("rk4_ties_upward", "if (0.5f * (float)(c[m] + c[m + 1]) < u) ++k;", "if (0.5f * (float)(c[m] + c[m + 1]) <= u) ++k;"),
    ("rk4_scale_divisor", "uint16_t h = orc_f32_to_f16_rne(a / 127.0f);\n    float sc = orc_f16_to_f32(h);",
     "uint16_t h = orc_f32_to_f16_rne(a / 96.0f);\n    float sc = orc_f16_to_f32(h);"),
    ("k4_nibble_order", "return byte * 8 + 4 * ((d % 8) / 4);", "return byte * 8 + 4 * (d % 2);"),
    ("bf16_ties_away", "if (rest > 0x8000u || (rest == 0x8000u && (hi & 1u))) hi += 1u;", "if (rest >= 0x8000u) hi += 1u;"),
    ("bf16_truncates", "if (rest > 0x8000u || (rest == 0x8000u && (hi & 1u))) hi += 1u;", "(void)rest;"),
    ("bf16_k_in_v_order", "page16[which ? orc_v_byte(slot, d, D) : orc_k_byte(slot, d, D)] = orc_f32_to_bf16_rne(x[d]);",
     "page16[orc_v_byte(slot, d, D)] = orc_f32_to_bf16_rne(x[d]);"),
]


def _build(tmp_path, text, name):
    src = tmp_path / f"{name}.c"
    src.write_text(text)
    so = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), "-o", str(so), str(src), "-lm"], check=True)
    return so


def _pins_pass(so):
    env = dict(os.environ, KVQ_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode == 0, r.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Every copy (the clean one and each planted mistake) built and run through the pins,
    several at a time (each run is its own process): name -> (pins passed, output tail)."""
    text = open(SRC).read()
    cases = {"clean": text}
    for name, orig, bad in MUTATIONS:
        assert text.count(orig) == 1, f"mutation site of {name} not found exactly once"
        cases[name] = text.replace(orig, bad)
    tmp = tmp_path_factory.mktemp("mutations")
    workers = max(1, min(8, (os.cpu_count() or 2) - 1))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        futs = {name: pool.submit(lambda n=name, t=src: _pins_pass(_build(tmp, t, n))) for name, src in cases.items()}
        return {name: f.result() for name, f in futs.items()}


def test_unmodified_copy_passes(outcomes):
    ok, out = outcomes["clean"]
    assert ok, out


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(outcomes, name):
    ok, _ = outcomes[name]
    assert not ok, f"the pins did not catch {name}"
