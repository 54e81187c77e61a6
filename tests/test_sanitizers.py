"""The C code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

The ScaledMaskSoftmax article (section 5.1) checks its kernel's host code with a memory
checker; the equivalent here covers the two C code bases that run on the host:
  - the oracle, built by gcc with both sanitizers, runs its pins, its argument checks and the
    parity checkers' own tests (every oracle entry point: forward, rows, backward, band,
    explicit mask, attention, codec);
  - libgtms.so, built by hipcc with the sanitizers on its host pass only (the kernels are
    compiled as usual and never launched here), runs the C ABI tests: every argument check
    and status code.
Each suite runs in a child Python whose first loaded library is the sanitizer runtime
(LD_PRELOAD); any sanitizer report stops it with a non-zero status.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def run_child(tests, preload, extra_env):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV, **extra_env)
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu", *tests], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    import oracle
    lib = str(tmp_path / "liboracle_sanitized.so")
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-O1", "-g", *SANITIZE, f"-I{oracle.HERE}",
                    oracle.SRC, "-o", lib, "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()
    out = run_child(["tests/test_oracle_pins.py", "tests/test_check_helpers.py"], asan,
                    {"GTMS_ORACLE_LIB": lib})
    print(out.strip().splitlines()[-1])


def clang_asan_runtime():
    base = "/opt/rocm/lib/llvm/lib/clang"
    for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def test_c_abi_host_code_under_sanitizers(tmp_path):
    runtime = clang_asan_runtime()
    if runtime is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from variable_length_causal_amd import build as hip_build
    lib = str(tmp_path / "libgtms_sanitized.so")
    host_only = [f for flag in SANITIZE for f in ("-Xarch_host", flag)]
    hip_build.build(extra_flags=host_only, out=lib)
    out = run_child(["tests/test_abi.py"], runtime, {"GTMS_LIBRARY": lib})
    print(out.strip().splitlines()[-1])
