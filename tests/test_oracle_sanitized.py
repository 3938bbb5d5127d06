"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
the CPU pin suites run in a child process against a sanitized build of
oracle/lfattn_oracle.c (gcc, every report fatal), so that an out-of-bounds
access, a use after free or undefined arithmetic in the oracle fails here
instead of silently moving the values every parity test is judged by."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lfattn_oracle.c")


def _gcc_runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                    "-pthread", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", SRC, "-o", lib, "-lm"], check=True)
    env = dict(os.environ)
    env.update(LFATTN_ORACLE_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    suites = ["tests/test_oracle_pins.py", "tests/test_oracle_pins_causal.py",
              "tests/test_oracle_pins_chunked.py", "tests/test_oracle_pins_global_proj.py",
              "tests/test_oracle_pins_grad.py"]
    proc = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", *suites], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=1200)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
