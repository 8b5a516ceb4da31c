"""Host code under the address and undefined-behaviour sanitizers (no GPU).

- The library's host shape logic (csrc/shape.cpp: descriptor checks, chunking, workspace
  sizes) is built with g++ -fsanitize=address,undefined beside a driver that sweeps
  ordinary and extreme arguments (tests/sanitize/shape_main.cpp).
- The CPU oracle (oracle/kvq_oracle.c) is built with gcc and the same sanitizers, and its
  pin suites run against that build in a child process (KVQ_ORACLE_LIB selects it; the
  sanitizer runtimes are preloaded into the interpreter).
Any sanitizer report aborts the program and fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_shape_logic_under_sanitizers(tmp_path):
    exe = tmp_path / "shape_main"
    subprocess.run(["g++", "-std=c++17"] + SAN + ["-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "paged_attention_quantized_kv_amd", "csrc", "shape.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "shape_main.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    sys.stdout.write(r.stdout + r.stderr)
    assert r.returncode == 0 and "shape ok" in r.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = tmp_path / "libkvq_oracle_san.so"
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"] + SAN +
                   ["-o", str(lib), os.path.join(ROOT, "oracle", "kvq_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, KVQ_ORACLE_LIB=str(lib), LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    suites = ["test_oracle_formats.py", "test_oracle_attention.py", "test_oracle_rk8v4.py", "test_oracle_rk4v4.py",
              "test_oracle_bf16.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", s) for s in suites], capture_output=True, text=True, env=env,
                       cwd=ROOT)
    sys.stdout.write(r.stdout[-3000:] + r.stderr[-3000:])
    assert r.returncode == 0, "oracle pins failed or a sanitizer fired under the sanitized build"
